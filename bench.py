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

With --op step it measures the single-token step (decode) instead, on a
2.7B-shaped layer with --decode-batch rows: one ssd_step launch per step, the
state resident in HBM, and prints a JSON line of the same form.  With --op bwd
it measures the backward pass (every input gradient for seeded upstream
gradients) on the named workload, in the same form.
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
COPY_BYTES = 256 << 20  # calibration copy: this many bytes read and written
PROFILES = os.path.join(ROOT, "profiles")


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
    ninit = inp.nseqs if inp.initial_states is not None else 0
    if name == "fused_prep":
        # dt in; prefix sums and dt' out; initial states copied into the hand-off ring
        return e * T * H + 2 * per_chunk_f32 + 2 * 4 * H * N * P * ninit
    if name == "fused":
        # the layer's compulsory bytes: the kernel does all of the pass but the
        # dt preparation (it reads the prefix sums in place of dt)
        return compulsory_bytes(wl, inp, with_final)
    if name == "stream":
        # the layer's compulsory bytes (x, B, C, dt in once, y out once, A and
        # D, initial and final states): the kernel does all of the pass but
        # the preparation, which reads dt, B and C once more to form the
        # per-chunk operands the kernel reads in their place
        return compulsory_bytes(wl, inp, with_final)
    if name == "stream_prep":
        # dt, B and C in; the prefix sums, the masked C B^T fragments and the
        # fp16 B and C operands out
        NI = Q // 16
        nfr = (NI // 2 + 1) * (NI // 2)
        bcg = inp.x.shape[0] * (nch // inp.x.shape[0]) * G
        return e * T * H + 2 * bc + per_chunk_f32 + bcg * nfr * 1024 + 2 * bc * 2 // e
    return 0


KERNEL_SOURCES = {"fused": "ssd_fused.hip", "fused_prep": "ssd_fused.hip", "step": "ssd_step.hip",
                  "bwd_chunk": "ssd_bwd.hip", "stream": "ssd_stream.hip",
                  "stream_prep": "ssd_stream.hip", "chunked": "ssd_chunked.hip"}


def kernel_sources_digest(kernel=None):
    """sha256 over the HIP source that builds `kernel` and the shared headers
    (every HIP source and header when the kernel is not named)."""
    import hashlib
    csrc = os.path.join(ROOT, "ssd_scan_amd", "csrc")
    own = KERNEL_SOURCES.get(kernel)
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith(".hpp") or (name.endswith(".hip") and own in (None, name)):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter on a copy
    of known size), or None when no summary exists or the kernel sources changed
    since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel sources sha256") != kernel_sources_digest(kernel):
        return None
    try:
        return float(fields["HBM bytes per launch (scaled)"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, budget_s):
    """Time the fp64 oracle on whole (sequence, head) streams of the workload until
    about budget_s of CPU work (going round the workload again when it takes
    less); report equivalent full-layer tokens/s."""
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
    while t_used < budget_s:
        start = done % len(order)
        pairs = order[start:start + batch]
        t0 = time.perf_counter()
        oracle.ssd_ref(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.dt_bias,
                       inp.initial_states, inp.cu_seqlens, softplus=inp.softplus,
                       dt_min=inp.dt_min, dt_max=inp.dt_max, pairs=pairs, want_final=False,
                       lib=lib)
        t_used += time.perf_counter() - t0
        tokens_heads += sum(lens[s] for s, _ in pairs)
        done += len(pairs)
        per_pair = t_used / done
        batch = max(cores, int((budget_s - t_used) / per_pair) // cores * cores)
    value = (tokens_heads / H) / t_used
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} (sequence, head) streams of the workload's {len(order)}, "
                      f"{tokens_heads} token-heads in {t_used:.1f} s, fp64 recurrence, "
                      f"OpenMP over streams, {model}"}


STEP_METRIC = "SSD decode step tokens/s, 2.7B-shaped layer (H80 P64 N128 G1, bf16), 1 GPU"


def step_main(args):
    """The single-token step: b rows of the 2.7B-shaped layer advance one token."""
    import numpy as np
    import torch

    import oracle
    import ssd_scan_amd as ssd

    b, H, P, N, G = args.decode_batch, 80, 64, 128, 1
    rng = np.random.default_rng(20240531 + 500)
    f32 = lambda *sh: rng.standard_normal(sh).astype(np.float32)
    x = f32(b, H, P)
    dtr = f32(b, H) - 4.6
    A = -np.exp(rng.uniform(0.0, np.log(16.0), H)).astype(np.float32)
    Bm = f32(b, G, N) / np.sqrt(N)
    Cm = f32(b, G, N) / np.sqrt(N)
    D = f32(H)
    S0 = f32(b, H, N, P)
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a).to(dev, torch.bfloat16)
    fl = lambda a: torch.from_numpy(a).to(dev, torch.float32)
    xd, dtd, Bd, Cd = bf(x), bf(dtr), bf(Bm), bf(Cm)
    Ad, Dd, S = fl(A), fl(D), fl(S0)
    y = torch.empty_like(xd)
    kw = dict(softplus=True, dt_min=1e-3, dt_max=0.1)
    stream = torch.cuda.current_stream()
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for k in range(args.warmup):
        if flush is not None:
            flush.fill_(k & 255)
        ssd.step(xd, dtd, Ad, Bd, Cd, S, Dd, out=y, **kw)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.fill_(k & 255)
        ev[k][0].record(stream)
        ssd.step(xd, dtd, Ad, Bd, Cd, S, Dd, out=y, **kw)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = [a.elapsed_time(z) for a, z in ev]
    step_s = float(np.mean(ms)) * 1e-3
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    # algorithmic bytes: the state in and out, x, dt, B, C in and y out, A and D
    kb = 2 * 4 * b * H * N * P + 2 * (2 * b * H * P + b * H + 2 * b * G * N) + 4 * 2 * H
    achieved = kb / step_s / 1e9
    out = {
        "metric": STEP_METRIC, "value": b / step_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": step_s * 1e3,
        "ms_median": float(np.median(ms)), "ms_min": float(np.min(ms)),
        "cold_caches": flush is not None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded, Mamba-2-shaped)",
        "config": {"workload": f"decode_2p7b_b{b}", "batch": b, "heads": H, "headdim": P,
                   "dstate": N, "ngroups": G},
        "roofline": {"bound": "hbm", "kernel": "step", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic("step", f"decode_2p7b_b{b}"),
                     "algorithmic_bytes": kb},
        "wall_s": t_wall,
    }
    if args.cpu_seconds > 0:
        # the oracle's step on the same rows (widened bf16 values), whole batch
        wid = lambda a: torch.from_numpy(a).to(torch.bfloat16).float().numpy()
        lib = oracle.load()
        t0 = time.perf_counter()
        oracle.ssd_ref_step(wid(x), wid(dtr), A, wid(Bm), wid(Cm), D, None, S0, lib=lib, **kw)
        dt_cpu = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": b / dt_cpu, "unit": "tokens/s",
                               "cores": oracle.num_threads(lib), "kind": "oracle",
                               "sample": f"all {b} rows x {H} heads, one step, fp64, "
                                         f"{dt_cpu:.2f} s"}
    print(json.dumps(out), flush=True)


BWD_METRIC = ("SSD bwd (all input gradients) tokens/s, 2.7B-shaped layer, L=4096, 1 GPU")
BWD_Q = 64            # chunk of the backward pass
BWD_MAX_EVENTS = 16


def bwd_head_block(H, G, Gc, nc, b, seq_terms, cus=256):
    """Heads per backward chunk workgroup, the library's rule: the largest of
    8, 4, 2 dividing the heads of every B and C group while the grid keeps at
    least 8 workgroups per CU, else 1; 1 when packed sequences carry states."""
    if seq_terms or H <= 0:
        return 1
    for k in (8, 4, 2):
        if (H // G) % k == 0 and (H // Gc) % k == 0 and H * nc * b // k >= 8 * cus:
            return k
    return 1


def bwd_kernel_bytes(name, wl, inp):
    """Bytes each backward kernel must move through its own interface, per
    launch (inputs read once, outputs written once; the dB / dC partials of
    each block of heads and the chunk states and adjoints are part of that
    interface: fp16 tiles with one 4-byte scale per 16 x 16 tile after the
    state walks (dense bf16 rows), fp32 otherwise)."""
    b, L, H, P = inp.x.shape
    N, G, Gc = inp.B.shape[3], inp.B.shape[2], inp.C.shape[2]
    e = 2 if wl.dtype == "bf16" else 4
    nc = -(-L // BWD_Q)
    tok = b * L
    seq_terms = inp.cu_seqlens is not None  # the binding always asks for the initial-state gradients
    hb = H // bwd_head_block(H, G, Gc, nc, b, seq_terms)  # head blocks
    states = b * nc * H * N * P * 4
    # the state walks (dense bf16 rows whose walk grid fills the 256 CUs), the
    # library's rule
    parts = (2 if N >= 64 else 1) if (P == 64 and N <= 128) else P // 32
    walked = wl.dtype == "bf16" and inp.cu_seqlens is None and H * b * parts >= 256
    wstates = b * nc * H * N * P * 2 + b * nc * H * (N * P // 256) * 4
    kstates = wstates if walked else states
    cs = 2 * b * H * nc * BWD_Q * 4
    return {
        "dt_cumsum": tok * H * e + cs,
        "state_walk": tok * H * P * e + tok * G * N * e + cs + wstates,
        "adjoint_walk": tok * H * P * e + tok * Gc * N * e + cs // 2 + wstates + b * H * N * P * 4 * 2,
        "chunk_state": tok * H * P * e + tok * G * N * e + cs + states,
        "state_passing": 2 * states,
        "chunk_adjoint": tok * H * P * e + tok * Gc * N * e + cs // 2 + states,
        "adjoint_passing": 3 * states + b * H * N * P * 4 * 2,
        "bwd_chunk": (3 * tok * H * P * e + tok * (G + Gc) * N * e + tok * H * e + cs
                      + 2 * kstates + 2 * tok * hb * N * 4 + tok * H * e),
        "group_sum_B": tok * hb * N * 4 + tok * G * N * e,
        "group_sum_C": tok * hb * N * 4 + tok * Gc * N * e,
        "head_sums": b * H * nc * 3 * 4 + 3 * H * 4,
    }.get(name)


def bwd_compulsory_bytes(wl, inp, with_dfinal):
    """The backward pass's compulsory I/O: x, dt, B, C, dy (and the final-state
    gradients, the initial states) read once; dx, ddt, dB, dC (and the initial
    state gradients) written once; A, D, dt_bias and their gradients."""
    b, L, H, P = inp.x.shape
    N, G, Gc = inp.B.shape[3], inp.B.shape[2], inp.C.shape[2]
    e = 2 if wl.dtype == "bf16" else 4
    T = b * L
    nst = (2 * inp.nseqs if inp.initial_states is not None else 0) + (inp.nseqs if with_dfinal else 0)
    return (e * (3 * T * H * P + 2 * T * H + 2 * T * (G + Gc) * N) + 4 * 6 * H
            + 4 * H * N * P * nst)


def bwd_flops(inp):
    """Matrix-core flops of the backward pass, causal count: per (row, head,
    64-token chunk) C B^T, dy x^T, and the dC, dx, dB in-chunk products over
    j <= i (3 Q^2 N + 2 Q^2 P), four state products in the chunk kernel and
    the chunk states and adjoints (12 Q N P)."""
    b, L, H, P = inp.x.shape
    N = inp.B.shape[3]
    Q = BWD_Q
    units = b * H * (-(-L // Q))
    return units * (3 * Q * Q * N + 2 * Q * Q * P + 12 * Q * N * P)


def bwd_main(args):
    """The backward pass: every input gradient of the layer for seeded dy and
    final-state gradients, inputs resident in HBM."""
    import numpy as np
    import torch

    import oracle
    import ssd_scan_amd as ssd
    import ssd_synth

    wl = ssd_synth.workloads()[args.workload]
    inp = ssd_synth.make(args.workload)
    if inp.cu_seqlens is not None and inp.initial_states is not None:
        raise SystemExit("the backward pass takes packed sequences without initial states")
    b, L, H, P = inp.x.shape
    N, G = wl.dstate, wl.ngroups
    dyn, dfn = ssd_synth.random_grads(wl.seed + 7, inp, with_dfinal=inp.cu_seqlens is None)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    t = lambda a, d=tdt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(
        device=dev, dtype=d)
    x, dt, B, C, dy = t(inp.x), t(inp.dt), t(inp.B), t(inp.C), t(dyn)
    A, D, dfin = t(inp.A, torch.float32), t(inp.D, torch.float32), t(dfn, torch.float32)
    init = t(inp.initial_states, torch.float32)
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    outs = [torch.empty_like(x), torch.empty_like(dt), torch.empty(H, **f32), torch.empty_like(B),
            torch.empty_like(C), torch.empty(H, **f32), torch.empty(H, **f32),
            None if cu is not None else torch.empty((b, H, N, P), **f32)]
    prob = ssd.make_problem(b, L, H, P, N, G, wl.chunk, bf16=wl.dtype == "bf16", softplus=True,
                            nseqs=0 if cu is None else inp.nseqs, dt_min=inp.dt_min,
                            dt_max=inp.dt_max)
    ws = torch.empty(max(ssd.bwd_workspace_size(prob), 1), dtype=torch.uint8, device=dev)
    lib = ssd.library()
    stream = torch.cuda.current_stream()
    ptr = lambda v: None if v is None else v.data_ptr()
    call_args = ([ctypes.byref(prob), ptr(x), ptr(dt), ptr(A), ptr(B), ptr(C), ptr(D), None,
                  ptr(init), ptr(cu), ptr(dy), ptr(dfin)] + [ptr(o) for o in outs]
                 + [ptr(ws), ws.numel(), ctypes.c_void_p(stream.cuda_stream)])
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(BWD_MAX_EVENTS)]
              for _ in range(args.steps)]
    for row in events:
        for ev in row:
            ev.record(stream)
    handles = [(ctypes.c_void_p * BWD_MAX_EVENTS)(*[ev.cuda_event for ev in row])
               for row in events]
    names = [(ctypes.c_char_p * BWD_MAX_EVENTS)() for _ in range(args.steps)]
    counts = [ctypes.c_int(0) for _ in range(args.steps)]
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for k in range(args.warmup):
        if flush is not None:
            flush.fill_(k & 255)
        st = lib.ssd_bwd(*call_args)
        if st != 0:
            raise ssd.SsdError(st, "ssd_bwd")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.fill_(k & 255)
        st = lib.ssd_bwd_events(*call_args, handles[k], names[k], BWD_MAX_EVENTS,
                                ctypes.byref(counts[k]))
        if st != 0:
            raise ssd.SsdError(st, "ssd_bwd")
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_ms = [events[k][0].elapsed_time(events[k][counts[k].value - 1])
               for k in range(args.steps)]
    ms_per_step = float(np.mean(step_ms))
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    per_kernel = {}
    for k in range(args.steps):
        for i in range(counts[k].value - 1):
            per_kernel.setdefault(names[k][i].decode(), []).append(
                events[k][i].elapsed_time(events[k][i + 1]))
    kernel_ms = {nm: float(np.mean(v)) for nm, v in per_kernel.items()}
    dominant = max(kernel_ms, key=kernel_ms.get)
    kb = bwd_kernel_bytes(dominant, wl, inp)
    achieved = kb / (kernel_ms[dominant] * 1e-3) / 1e9
    step_s = ms_per_step * 1e-3
    flops = bwd_flops(inp)
    out = {
        "metric": BWD_METRIC, "value": b * L / step_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "ms_median": float(np.median(step_ms)), "ms_min": float(np.min(step_ms)),
        "cold_caches": flush is not None, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic (seeded, Mamba-2-shaped; see ssd_synth.py)",
        "config": {"workload": wl.name, "batch": b, "seqlen": L, "heads": H, "headdim": P,
                   "dstate": N, "ngroups": G, "chunk": BWD_Q, "pass": "backward",
                   "packed_sequences": 0 if cu is None else inp.nseqs},
        "tflops": flops / step_s / 1e12,
        "pct_mfma_peak": 100.0 * flops / step_s / 1e12 / MFMA_PEAK_TFLOPS[wl.dtype],
        "kernel_ms": kernel_ms,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(dominant, wl.name), "algorithmic_bytes": kb},
        # the whole pass against its compulsory I/O (the kernels' interfaces
        # above include the fp32 intermediates the schedule chooses to move)
        "op_compulsory_bytes": bwd_compulsory_bytes(wl, inp, dfn is not None),
        "op_roofline_frac": bwd_compulsory_bytes(wl, inp, dfn is not None) / step_s / 1e9 / HBM_PEAK_GBS,
        "wall_s": t_wall,
    }
    if args.cpu_seconds > 0 and cu is None:
        # the oracle's gradients of the first row, for as many heads as the budget allows
        wid = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).float().numpy() \
            if wl.dtype == "bf16" else a
        lib_o = oracle.load()
        nh, done_tok, spent = 1, 0.0, 0.0
        while spent < args.cpu_seconds:
            hs = np.arange(nh) % H
            t0 = time.perf_counter()
            oracle.ssd_ref_bwd(wid(inp.x[:1][:, :, hs]), wid(inp.dt[:1][:, :, hs]), inp.A[hs],
                               wid(inp.B[:1]), wid(inp.C[:1]), wid(dyn[:1][:, :, hs]),
                               inp.D[hs], None,
                               None if inp.initial_states is None else inp.initial_states[:1][:, hs], None,
                               dfn[:1][:, hs], softplus=True, dt_min=inp.dt_min,
                               dt_max=inp.dt_max, lib=lib_o)
            spent += time.perf_counter() - t0
            done_tok += L * nh / H
            nh = min(2 * nh, 4 * H)
        out["cpu_baseline"] = {"value": done_tok / spent, "unit": "tokens/s",
                               "cores": oracle.num_threads(lib_o), "kind": "oracle",
                               "sample": f"row 0, L={L}, {done_tok * H / L:.0f} (head) streams "
                                         f"of the backward recurrence, fp64, {spent:.1f} s"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mamba2_2p7b")
    ap.add_argument("--algo", default="auto", choices=["auto", "chunked", "fused", "stream"])
    ap.add_argument("--final-states", action="store_true", help="also return final states")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU work budget of the oracle baseline (0 disables it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 256 MB device to device three times "
                         "(the reference kernel for scaling HBM counters)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the untimed 512 MB write before each step that evicts L2 and MALL")
    ap.add_argument("--op", default="fwd", choices=["fwd", "step", "bwd"],
                    help="fwd: the forward pass (default); step: the single-token step; "
                         "bwd: the backward pass (all input gradients)")
    ap.add_argument("--decode-batch", type=int, default=256, help="rows of the step benchmark")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU; run it with --gpus 1"}))
        sys.exit(2)

    if args.op == "step":
        step_main(args)
        return
    if args.op == "bwd":
        bwd_main(args)
        return

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

    # Each step starts from cold caches: an untimed 512 MB write (twice the
    # MALL) precedes it on the same stream.  A step's time runs from the event
    # before its first launch to the event after its last one.
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for k in range(args.warmup):
        if flush is not None:
            flush.fill_(k & 255)
        st = lib.ssd_fwd(*call_args)
        if st != 0:
            raise ssd.SsdError(st)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(args.steps):
        if flush is not None:
            flush.fill_(k & 255)
        st = lib.ssd_fwd_events(*call_args, handles[k], names[k], MAX_EVENTS,
                                ctypes.byref(counts[k]))
        if st != 0:
            raise ssd.SsdError(st)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_ms = [events[k][0].elapsed_time(events[k][counts[k].value - 1])
               for k in range(args.steps)]
    ms_per_step = float(np.mean(step_ms))

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

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
        "ms_median": float(np.median(step_ms)),
        "ms_min": float(np.min(step_ms)),
        "cold_caches": flush is not None,
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
                     "traffic": measured_traffic(dominant, wl.name), "algorithmic_bytes": kb},
        "wall_s": t_wall,
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
