"""Shared helpers of the GPU parity tests: move seeded inputs to the device, run
the HIP path through the C ABI binding, run the oracle on the same values, and
compare them with the error measure and tolerances of the method.

Error measure: max_i |y_i - ref_i| / max(|ref_i|, rms(ref)), over y and over the
final states separately.  Tolerances: 1e-4 for fp32 inputs, 2e-2 for bf16
inputs (fp32 accumulation).
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

import oracle
from checkers import rel_err

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def record(case: str, **errs):
    """Print the observed errors of a case and, when SSD_MARGIN_LOG names a
    file, append them to it as one JSON line (the margin table is built from
    these)."""
    vals = {k: (None if v is None else float(v)) for k, v in errs.items()}
    say("margin " + case + ": " + ", ".join(
        f"{k} {v:.3e}" for k, v in vals.items() if v is not None))
    path = os.environ.get("SSD_MARGIN_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": case, **vals}) + "\n")


def to_device(inp):
    import torch

    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32

    def cvt(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(
            device="cuda", dtype=dt)

    def f32(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

    cu = None if inp.cu_seqlens is None else torch.from_numpy(
        np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)).to("cuda")
    return dict(x=cvt(inp.x), dt=cvt(inp.dt), A=f32(inp.A), B=cvt(inp.B), C=cvt(inp.C),
                D=f32(inp.D), dt_bias=f32(inp.dt_bias), initial_states=f32(inp.initial_states),
                cu_seqlens=cu)


def run_gpu(inp, algo="auto", chunk=None, want_final=True, dev=None):
    import torch

    import ssd_scan_amd as ssd

    dev = dev or to_device(inp)
    kw = dict(chunk_size=chunk or inp.chunk, softplus=inp.softplus, scales_input=inp.scales_input,
              dt_min=inp.dt_min, dt_max=inp.dt_max, algo=algo)
    if want_final:
        y, fin = ssd.fwd(**dev, **kw, return_final_states=True)
    else:
        y, fin = ssd.fwd(**dev, **kw), None
    torch.cuda.synchronize()
    yh = y.float().cpu().numpy().astype(np.float64)
    fh = None if fin is None else fin.cpu().numpy().astype(np.float64)
    return yh, fh


def fwd_into(inp, algo):
    """ssd_fwd into a preallocated y; returns (y on the host, the SsdError or None)."""
    import torch

    import ssd_scan_amd as ssd

    dev = to_device(inp)
    y = torch.zeros_like(dev["x"])
    err = None
    try:
        ssd.fwd(**dev, chunk_size=inp.chunk, softplus=inp.softplus, scales_input=inp.scales_input,
                dt_min=inp.dt_min, dt_max=inp.dt_max, algo=algo, out=y)
    except ssd.SsdError as e:
        err = e
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), err


def run_oracle(inp, pairs=None, want_final=True):
    return oracle.ssd_ref(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.dt_bias,
                          inp.initial_states, inp.cu_seqlens, softplus=inp.softplus,
                          scales_input=inp.scales_input, dt_min=inp.dt_min, dt_max=inp.dt_max,
                          pairs=pairs, want_final=want_final)


def stream_slices(inp, pairs):
    """(row, token slice, head) of each (sequence, head) pair."""
    out = []
    for s, h in pairs:
        if inp.cu_seqlens is None:
            out.append((s, slice(0, inp.x.shape[1]), h))
        else:
            out.append((0, slice(int(inp.cu_seqlens[s]), int(inp.cu_seqlens[s + 1])), h))
    return out


def compare(inp, y, fin, yr, fr, pairs=None):
    """Returns (err_y, err_final) over all streams or over the sampled pairs."""
    if pairs is None:
        ey = rel_err(y, yr)
        ef = None if (fin is None or fr is None) else rel_err(fin, fr)
        return ey, ef
    got, ref, gf, rf = [], [], [], []
    for (row, sl, h), (s, _) in zip(stream_slices(inp, pairs), pairs):
        got.append(y[row, sl, h].ravel())
        ref.append(yr[row, sl, h].ravel())
        if fin is not None and fr is not None:
            gf.append(fin[s, h].ravel())
            rf.append(fr[s, h].ravel())
    ey = rel_err(np.concatenate(got), np.concatenate(ref))
    ef = rel_err(np.concatenate(gf), np.concatenate(rf)) if gf else None
    return ey, ef
