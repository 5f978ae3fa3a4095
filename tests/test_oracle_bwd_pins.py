"""Pins of the oracle's backward pass (``oracle.ssd_ref_bwd``), on the CPU.

The gradients are checked against two things other than the oracle's own
adjoint loop: central differences of the forward oracle (itself pinned in
test_oracle_pins.py), and reverse-mode differentiation, by PyTorch autograd in
float64, of the layer written in its quadratic matrix form ("Transformers are
SSMs", section 3.1 / 3.3: y = M x with M[t,u] = (C_t . B_u) a_{u+1} ... a_t,
section 5.3's dual form) with the initial state's decayed readout, the final
state, the D skip, shared B/C heads (section 7.1 / 7.2) and packed sequences
(section 8.3).  The loss is sum(dy * y) + sum(dfinal * final).
"""
import numpy as np
import pytest
import torch

import oracle

FIELDS = ("x", "dt", "A", "B", "C", "D", "dt_bias", "init")


def _case(seed, b, L, H, P, N, G, Gc, cu=None, softplus=True, scales=False, dt_min=0.0,
          dt_max=np.inf, with_init=True):
    """Tiny case with decays a = exp(dt' A) in about [0.4, 0.97], some tokens on
    either side of the clamp, and no value within 1e-2 of a clamp edge."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    nseq = b if cu is None else len(cu) - 1
    c = dict(
        x=rng.standard_normal((b, L, H, P)).astype(f32),
        A=(-np.exp(rng.uniform(0.0, np.log(4.0), H))).astype(f32),
        B=(rng.standard_normal((b, L, G, N)) * 0.7).astype(f32),
        C=(rng.standard_normal((b, L, Gc, N)) * 0.7).astype(f32),
        D=rng.standard_normal(H).astype(f32),
        dt_bias=(rng.standard_normal(H) * 0.3).astype(f32),
        init=rng.standard_normal((nseq, H, N, P)).astype(f32) if with_init else None,
    )
    raw = rng.uniform(-3.0, 0.5, (b, L, H)) if softplus else rng.uniform(0.02, 0.3, (b, L, H))
    act = lambda v: np.logaddexp(v, 0.0) if softplus else v  # noqa: E731
    for _ in range(50):  # move values off the clamp edges
        a = act(raw + c["dt_bias"][None, None, :].astype(np.float64))
        near = (np.abs(a - dt_min) < 1e-2) | (np.abs(a - dt_max) < 1e-2)
        if not near.any():
            break
        raw = np.where(near, raw + 0.05, raw)
    c["dt"] = raw.astype(f32)
    c["dy"] = rng.standard_normal((b, L, H, P)).astype(f32)
    c["dfin"] = rng.standard_normal((nseq, H, N, P)).astype(f32)
    c["opts"] = dict(softplus=softplus, scales_input=scales, dt_min=dt_min, dt_max=dt_max)
    c["cu"] = None if cu is None else np.asarray(cu, np.int32)
    return c


FD_CASES = [
    dict(seed=1, b=2, L=6, H=2, P=3, N=2, G=1, Gc=2, dt_max=0.3),
    dict(seed=2, b=2, L=5, H=2, P=2, N=3, G=2, Gc=1, softplus=False, scales=True, dt_min=0.05,
         dt_max=0.25),
    dict(seed=3, b=1, L=7, H=2, P=2, N=2, G=1, Gc=1, cu=[0, 2, 2, 7], scales=True, dt_max=0.35),
]


def _loss(c, lib=None, **over):
    v = {k: c[k] for k in FIELDS}
    v.update(over)
    y, fin = oracle.ssd_ref(v["x"], v["dt"], v["A"], v["B"], v["C"], v["D"], v["dt_bias"], v["init"],
                            c["cu"], lib=lib, **c["opts"])
    return float(np.sum(c["dy"] * y) + np.sum(c["dfin"] * fin))


def _grads(c, lib=None):
    return oracle.ssd_ref_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["dy"], c["D"], c["dt_bias"],
                              c["init"], c["cu"], c["dfin"], lib=lib, **c["opts"])


KEY = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "dt_bias": "ddt_bias",
       "init": "dinit"}


@pytest.mark.parametrize("spec", FD_CASES, ids=lambda s: f"seed{s['seed']}")
def test_bwd_matches_central_differences(oracle_lib, spec):
    c = _case(**spec)
    g = _grads(c, oracle_lib)
    h = np.float32(2.0 ** -10)
    for name in FIELDS:
        base = c[name]
        num = np.zeros(base.shape)
        flat = base.reshape(-1)
        for i in range(flat.size):
            hi, lo = flat.copy(), flat.copy()
            hi[i] += h
            lo[i] -= h
            step = float(hi[i]) - float(lo[i])
            num.reshape(-1)[i] = (_loss(c, oracle_lib, **{name: hi.reshape(base.shape)})
                                  - _loss(c, oracle_lib, **{name: lo.reshape(base.shape)})) / step
        ana = g[KEY[name]]
        scale = max(np.max(np.abs(num)), 1e-3)
        err = np.max(np.abs(ana - num)) / scale
        assert err < 2e-5, f"{name}: analytic vs central differences rel err {err:.2e}"


def _torch_loss(t, c):
    """sum(dy * y) + sum(dfinal * final) of the quadratic (matrix) form."""
    x, dtr, A, B, C, D, bias, init = (t[k] for k in FIELDS)
    o = c["opts"]
    b, L, H, P = x.shape
    G, Gc = B.shape[2], C.shape[2]
    pre = dtr + bias[None, None, :]
    act = torch.logaddexp(pre, torch.zeros_like(pre)) if o["softplus"] else pre
    dte = torch.clamp(act, o["dt_min"], o["dt_max"] if np.isfinite(o["dt_max"]) else None)
    dy = torch.from_numpy(c["dy"].astype(np.float64))
    dfin = torch.from_numpy(c["dfin"].astype(np.float64))
    if c["cu"] is None:
        streams = [(s, s, 0, L) for s in range(b)]
    else:
        cu = c["cu"]
        streams = [(s, 0, int(cu[s]), int(cu[s + 1])) for s in range(len(cu) - 1)]
    loss = torch.zeros((), dtype=torch.float64)
    for s, row, t0, t1 in streams:
        T = t1 - t0
        for h in range(H):
            S0 = init[s, h]
            if T == 0:
                loss = loss + (dfin[s, h] * S0).sum()
                continue
            lg = dte[row, t0:t1, h] * A[h]
            cs = torch.cumsum(lg, 0)
            seg = cs[:, None] - cs[None, :]
            mask = torch.tril(torch.ones(T, T, dtype=torch.bool))
            decay = torch.exp(seg.masked_fill(~mask, -1e30))
            scale = dte[row, t0:t1, h] if o["scales_input"] else torch.ones(T, dtype=torch.float64)
            Bs = B[row, t0:t1, h // (H // G)]
            Cs = C[row, t0:t1, h // (H // Gc)]
            xs = x[row, t0:t1, h]
            M = (Cs @ Bs.T) * decay * scale[None, :]
            ys = M @ xs + D[h] * xs + torch.exp(cs)[:, None] * (Cs @ S0)
            fin = (Bs * (decay[T - 1] * scale)[:, None]).T @ xs + torch.exp(cs[T - 1]) * S0
            loss = loss + (dy[row, t0:t1, h] * ys).sum() + (dfin[s, h] * fin).sum()
    return loss


AUTOGRAD_CASES = [
    dict(seed=11, b=2, L=33, H=4, P=5, N=3, G=2, Gc=1, dt_max=0.3),
    dict(seed=12, b=1, L=29, H=4, P=3, N=4, G=1, Gc=4, softplus=False, scales=True, dt_min=0.05,
         dt_max=0.25),
    dict(seed=13, b=1, L=40, H=2, P=4, N=2, G=1, Gc=2, cu=[0, 9, 9, 30, 40], scales=True,
         dt_max=0.35),
    dict(seed=14, b=3, L=17, H=2, P=3, N=2, G=2, Gc=2, with_init=False),
]


@pytest.mark.parametrize("spec", AUTOGRAD_CASES, ids=lambda s: f"seed{s['seed']}")
def test_bwd_matches_autograd_of_quadratic_form(oracle_lib, spec):
    c = _case(**spec)
    g = _grads(c, oracle_lib)
    nseq = c["dfin"].shape[0]
    H, N, P = c["x"].shape[2], c["B"].shape[3], c["x"].shape[3]
    t = {}
    for k in FIELDS:
        v = c[k] if c[k] is not None else np.zeros((nseq, H, N, P), np.float32)
        t[k] = torch.tensor(v.astype(np.float64), requires_grad=True)
    if c["init"] is None:
        t["init"].requires_grad_(False)
    loss = _torch_loss(t, c)
    wrt = [k for k in FIELDS if t[k].requires_grad]
    ref = dict(zip(wrt, torch.autograd.grad(loss, [t[k] for k in wrt])))
    for k in wrt:
        r = ref[k].numpy()
        err = np.max(np.abs(g[KEY[k]] - r)) / max(np.max(np.abs(r)), 1e-12)
        assert err < 1e-10, f"{k}: oracle vs autograd of the quadratic form rel err {err:.2e}"
    if c["init"] is None:  # gradient with respect to a zero initial state is still defined
        t["init"].requires_grad_(True)
        (ri,) = torch.autograd.grad(_torch_loss(t, c), [t["init"]])
        assert np.max(np.abs(g["dinit"] - ri.numpy())) <= 1e-10 * max(np.max(np.abs(ri.numpy())), 1)


def test_bwd_without_dfinal_is_zero_dfinal(oracle_lib):
    c = _case(seed=21, b=2, L=9, H=2, P=2, N=2, G=1, Gc=1)
    a = oracle.ssd_ref_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], c["dy"], c["D"], c["dt_bias"],
                           c["init"], None, None, lib=oracle_lib, **c["opts"])
    c["dfin"] = np.zeros_like(c["dfin"])
    b = _grads(c, oracle_lib)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
