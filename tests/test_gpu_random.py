"""Seeded random shapes through every schedule that takes them, against the
fp64 oracle (forward) and the oracle's gradients (backward).

Each case draws its shape and options from a fixed seed: batch rows or packed
sequences (with empty ones and starts anywhere), sequence length (ragged
against the chunk), heads and B / C group counts (including separate C
groups), every supported N, P, Q and storage type, initial states, D or not,
dt bias, softplus or not and the input-scaling flag.  The hand-written cases
of the other files pin each feature on purpose; these cover combinations
nobody picked.
"""
import numpy as np
import pytest

import oracle
import ssd_synth
from checkers import rel_err
from parity import TOL, compare, record, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


def draw_case(k, for_bwd=False):
    r = np.random.default_rng(7000 + 31 * k + (5 if for_bwd else 0))
    dtype = "bf16" if r.random() < 0.7 else "f32"
    P = 64 if r.random() < 0.7 else 128
    Ns = [16, 32, 64, 128, 256]
    lim = (16384 if dtype == "bf16" else 8192) if for_bwd else (1 << 30 if dtype == "bf16" else 16384)
    N = int(r.choice([n for n in Ns if n * P <= lim]))
    Q = int(r.choice([64, 128, 256]))
    H = int(r.integers(1, 7))
    G = int(r.choice(_divisors(H)))
    Gc = int(r.choice(_divisors(H))) if r.random() < 0.2 else None
    packed = r.random() < 0.3
    if packed:
        n = int(r.integers(1, 8))
        lengths = [int(v) if r.random() > 0.15 else 0 for v in r.integers(1, 400, size=n)]
        L = sum(lengths)
        if L == 0:
            lengths[0] = L = 1
        b = 1
    else:
        lengths = None
        b = int(r.integers(1, 4))
        L = int(r.integers(1, 1200))
    inp = ssd_synth.random_case(9000 + k + (500 if for_bwd else 0), b, L, H, P, N, G, chunk=Q,
                                dtype=dtype, with_init=r.random() < 0.5, lengths=lengths,
                                with_D=r.random() < 0.7, Gc=Gc)
    if r.random() < 0.3:
        inp.dt_bias = r.normal(0.0, 1.0, size=H).astype(np.float32)
    if r.random() < 0.1:
        inp.softplus = False
        inp.dt_bias = np.full(H, 4.7, np.float32)
        inp.dt_min, inp.dt_max = 0.0, 0.2
    inp.scales_input = bool(r.random() < 0.2)
    desc = (f"{dtype} b{b} L{L} H{H} P{P} N{N} G{G} Gc{Gc or G} Q{Q}"
            f"{' packed ' + str(lengths) if packed else ''} init={inp.initial_states is not None}"
            f" D={inp.D is not None} bias={inp.dt_bias is not None} softplus={inp.softplus}"
            f" scaled={inp.scales_input}")
    return inp, desc


def _schedules(inp):
    bf16, P64 = inp.dtype == "bf16", inp.x.shape[3] == 64
    out = ["auto", "chunked"]
    if bf16 and P64 and inp.B.shape[3] <= 128:
        out.append("fused")
    if bf16 and P64 and inp.cu_seqlens is None and inp.B.shape[2] == inp.C.shape[2]:
        out.append("stream")
    return out


@pytest.mark.parametrize("k", range(160))
def test_random_forward(k):
    inp, desc = draw_case(k)
    yr, fr = run_oracle(inp)
    tol = TOL[inp.dtype]
    for algo in _schedules(inp):
        say(f"random fwd {k} {algo}: {desc}")
        y, fin = run_gpu(inp, algo=algo)
        ey, ef = compare(inp, y, fin, yr, fr)
        record(f"random fwd {k} {algo}", y=ey, final=ef)
        assert np.isfinite(y).all() and np.isfinite(fin).all(), (algo, desc)
        assert ey < tol and ef < tol, (algo, desc, ey, ef)


@pytest.mark.parametrize("k", range(64))
def test_random_backward(k):
    import ssd_scan_amd as ssd
    from parity import to_device

    inp, desc = draw_case(k, for_bwd=True)
    dy, dfin = ssd_synth.random_grads(11000 + k, inp, with_dfinal=inp.initial_states is not None)
    say(f"random bwd {k}: {desc}")
    dev = to_device(inp)
    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    g = ssd.bwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"],
                torch.from_numpy(dy).to("cuda", tdt), D=dev["D"], dt_bias=dev["dt_bias"],
                initial_states=dev["initial_states"],
                d_final_states=None if dfin is None else torch.from_numpy(dfin).to("cuda"),
                cu_seqlens=dev["cu_seqlens"], softplus=inp.softplus,
                scales_input=inp.scales_input, dt_min=inp.dt_min, dt_max=inp.dt_max)
    torch.cuda.synchronize()
    ref = oracle.ssd_ref_bwd(inp.x, inp.dt, inp.A, inp.B, inp.C, dy, inp.D, inp.dt_bias,
                             inp.initial_states, inp.cu_seqlens, dfin, softplus=inp.softplus,
                             scales_input=inp.scales_input, dt_min=inp.dt_min,
                             dt_max=inp.dt_max, want_dinit=inp.initial_states is not None)
    tol = TOL[inp.dtype]
    keys = ["dx", "ddt", "dA", "dB", "dC", "ddt_bias"] + (["dD"] if inp.D is not None else [])
    if inp.initial_states is not None:
        keys.append("dinit")
    errs = {}
    for key in keys:
        got = g[key].float().cpu().numpy().astype(np.float64)
        errs[key] = rel_err(got, ref[key])
    record(f"random bwd {k}", **errs)
    for key, e in errs.items():
        assert np.isfinite(e) and e < tol, (key, e, desc)
