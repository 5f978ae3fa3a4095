"""Offsets past 2^31 elements: x and y of more than 2^31 elements each, every
schedule, sampled (row, head) streams against the oracle.

b2 L550123 H32 P64 N64 G1 Q256 bf16: x has 2 253 303 808 elements, so every
offset of row 1 past token 498 453 exceeds the int32 range; the sampled heads
of row 1 reach the last element.  Inputs are drawn on the device with the
workload distributions (ssd_synth.large_case_device); the oracle runs the
token recurrence of the sampled streams in full on the host.
"""
from __future__ import annotations

import numpy as np
import pytest

import ssd_synth
from parity import TOL, record, run_oracle, say

pytestmark = pytest.mark.gpu

SHAPE = dict(batch=2, seqlen=550123, H=32, P=64, N=64)
HEADS = [0, 17, 31]


@pytest.fixture(scope="module")
def large():
    import torch

    say(f"large case {SHAPE}")
    dev = ssd_synth.large_case_device(20240531 + 900, SHAPE["batch"], SHAPE["seqlen"], SHAPE["H"],
                                      SHAPE["P"], SHAPE["N"])
    assert dev["x"].numel() > 2 ** 31
    host = ssd_synth.host_subset(dev, HEADS)
    say("large case: oracle on the sampled heads")
    yr, fr = run_oracle(host)
    yield dev, host, yr, fr
    del dev
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo", ["auto", "stream", "fused", "chunked"])
def test_offsets_past_2_31_elements(large, algo):
    import torch

    import ssd_scan_amd as ssd

    dev, host, yr, fr = large
    say(f"large case algo={algo}")
    y, fin = ssd.fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], D=dev["D"], chunk_size=256,
                     softplus=True, dt_min=ssd_synth.DT_MIN, dt_max=ssd_synth.DT_MAX, algo=algo,
                     return_final_states=True)
    idx = torch.tensor(HEADS, device=y.device)
    ys = y.index_select(2, idx).float().cpu().numpy().astype(np.float64)
    fs = fin.index_select(1, idx).cpu().numpy().astype(np.float64)
    del y, fin
    from checkers import rel_err

    ey, ef = rel_err(ys, yr), rel_err(fs, fr)
    # the rows' tails, where the offsets pass 2^31, on their own
    tail = slice(SHAPE["seqlen"] - 60000, None)
    et = rel_err(ys[1, tail], yr[1, tail])
    record(f"large b2 L550123 H32 N64 heads {HEADS} algo={algo}", y=ey, y_row1_tail=et, final=ef)
    assert np.isfinite(ys).all() and np.isfinite(fs).all()
    assert ey < TOL["bf16"] and et < TOL["bf16"] and ef < TOL["bf16"]


def test_bwd_offsets_past_2_31_elements(large):
    """The backward pass on the same case: dx, ddt, dA and dD of the sampled
    heads against the oracle's gradients of those heads (each depends on its
    own head's stream only; dB and dC sum over every head and are compared at
    full size on the 2.7B-shaped layer instead)."""
    import torch

    import oracle
    import ssd_scan_amd as ssd

    dev, host, _, _ = large
    say("large case backward")
    dy = ssd_synth.large_grad_device(20240531 + 901, dev["x"])
    g = ssd.bwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dy, D=dev["D"], softplus=True,
                dt_min=ssd_synth.DT_MIN, dt_max=ssd_synth.DT_MAX)
    idx = torch.tensor(HEADS, device=dy.device)
    dys = dy.index_select(2, idx).float().cpu().numpy()
    got = {"dx": g["dx"].index_select(2, idx), "ddt": g["ddt"].index_select(2, idx),
           "dA": g["dA"][idx], "dD": g["dD"][idx]}
    got = {k: v.float().cpu().numpy().astype(np.float64) for k, v in got.items()}
    del g, dy
    torch.cuda.empty_cache()
    say("large case backward: oracle on the sampled heads")
    ref = oracle.ssd_ref_bwd(host.x, host.dt, host.A, host.B, host.C, dys, host.D, softplus=True,
                             dt_min=host.dt_min, dt_max=host.dt_max, want_dinit=False)
    from checkers import rel_err

    errs = {k: rel_err(got[k], ref[k]) for k in got}
    tail = slice(SHAPE["seqlen"] - 60000, None)
    errs["dx_row1_tail"] = rel_err(got["dx"][1, tail], ref["dx"][1, tail])
    record(f"large bwd b2 L550123 H32 N64 heads {HEADS}", **errs)
    for k, e in errs.items():
        assert np.isfinite(e) and e < TOL["bf16"], f"{k}: {e:.3e}"


def test_step_state_past_2_31_elements():
    """The single-token step on a state of more than 2^31 elements (b4096 H80
    N128 P64 fp32, 10.7 GB): y and the new state of sampled rows against the
    oracle's step from the same state."""
    import torch

    import oracle
    import ssd_scan_amd as ssd

    b, H, P, N = 4096, 80, 64, 128
    say(f"large step b{b} H{H} N{N} P{P}")
    dev = ssd_synth.large_case_device(20240531 + 902, b, 1, H, P, N)
    state = ssd_synth.large_grad_device(20240531 + 903, torch.empty((b, H, N, P), device="cuda"))
    assert state.numel() > 2 ** 31 and state.is_contiguous()
    rows = [0, 2047, 4095]
    ridx = torch.tensor(rows, device="cuda")
    s0 = state.index_select(0, ridx).cpu().numpy()
    y = ssd.step(dev["x"][:, 0], dev["dt"][:, 0], dev["A"], dev["B"][:, 0], dev["C"][:, 0], state,
                 D=dev["D"], softplus=True, dt_min=ssd_synth.DT_MIN, dt_max=ssd_synth.DT_MAX)
    ys = y.index_select(0, ridx).float().cpu().numpy().astype(np.float64)
    s1 = state.index_select(0, ridx).cpu().numpy().astype(np.float64)
    f = lambda t: t.index_select(0, ridx).float().cpu().numpy()
    yr, sr = oracle.ssd_ref_step(f(dev["x"][:, 0]), f(dev["dt"][:, 0]), dev["A"].cpu().numpy(),
                                 f(dev["B"][:, 0]), f(dev["C"][:, 0]), dev["D"].cpu().numpy(),
                                 None, s0, softplus=True, dt_min=ssd_synth.DT_MIN,
                                 dt_max=ssd_synth.DT_MAX)
    del dev, state, y
    torch.cuda.empty_cache()
    from checkers import rel_err

    ey, es = rel_err(ys, yr), rel_err(s1, sr)
    record(f"large step b{b} H{H} N{N} rows {rows}", y=ey, state=es)
    assert ey < TOL["bf16"] and es < TOL["bf16"]
