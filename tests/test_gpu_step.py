"""GPU parity of the single-token step (recurrent / decode mode) against the
fp64 oracle's step, through the C ABI.

Each case draws the workload distributions for one token per row plus a state,
runs ``ssd_step`` and the oracle's one-token recurrence from the same state,
and compares y and the new state with the error measure and tolerances of the
forward pass.  A second test hands the final states of a forward pass to the
step and checks the next token against a longer oracle run.
"""
import numpy as np
import pytest

import oracle
import ssd_synth
from checkers import rel_err
from parity import TOL, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [
    dict(name="bf16_P64_N128_G1", seed=201, b=4, H=8, P=64, N=128, G=1, dtype="bf16"),
    dict(name="bf16_P128_N256_G2", seed=202, b=2, H=4, P=128, N=256, G=2, dtype="bf16"),
    dict(name="f32_P64_N16_G4", seed=203, b=3, H=4, P=64, N=16, G=4, dtype="f32"),
    dict(name="f32_P128_N64_scaled_bias", seed=204, b=2, H=6, P=128, N=64, G=3, dtype="f32",
         scales_input=True, bias=0.7),
    dict(name="bf16_P64_N32_odd_rows", seed=205, b=5, H=3, P=64, N=33, G=1, dtype="bf16"),
    dict(name="bf16_P64_N64_multi_contract", seed=206, b=3, H=4, P=64, N=64, G=1, Gc=4,
         dtype="bf16"),
    dict(name="f32_P128_N16_multi_expand", seed=207, b=2, H=4, P=128, N=16, G=4, Gc=1,
         dtype="f32"),
]


def _draw(c):
    """One token per row from the workload distributions, and a random state."""
    inp = ssd_synth.random_case(c["seed"], c["b"], 1, c["H"], c["P"], c["N"], c["G"], chunk=64,
                                dtype=c["dtype"], with_init=True, Gc=c.get("Gc"))
    x, dt, B, C = inp.x[:, 0], inp.dt[:, 0], inp.B[:, 0], inp.C[:, 0]
    bias = np.full(c["H"], c.get("bias", 0.0), np.float32) if "bias" in c else None
    return inp, x, dt, B, C, bias


def _dev(a, dtype):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype)


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
@pytest.mark.parametrize("with_D", [True, False], ids=["D", "noD"])
def test_step_matches_oracle(c, with_D):
    import ssd_scan_amd as ssd

    inp, x, dt, B, C, bias = _draw(c)
    D = inp.D if with_D else None
    scales = c.get("scales_input", False)
    tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    state = _dev(inp.initial_states, torch.float32)
    say(f"step {c['name']} D={with_D}")
    y = ssd.step(_dev(x, tdt), _dev(dt, tdt), _dev(inp.A, torch.float32), _dev(B, tdt),
                 _dev(C, tdt), state, _dev(D, torch.float32), _dev(bias, torch.float32),
                 softplus=True, scales_input=scales, dt_min=inp.dt_min, dt_max=inp.dt_max)
    torch.cuda.synchronize()
    yr, sr = oracle.ssd_ref_step(x, dt, inp.A, B, C, D, bias, inp.initial_states, softplus=True,
                                 scales_input=scales, dt_min=inp.dt_min, dt_max=inp.dt_max)
    ey = rel_err(y.float().cpu().numpy(), yr)
    es = rel_err(state.cpu().numpy(), sr)
    assert ey < TOL[c["dtype"]], f"y error {ey:.3e}"
    # the state is updated in fp32 from the same values: fp32 rounding only
    assert es < 1e-5, f"state error {es:.3e}"


@pytest.mark.parametrize("algo", ["auto", "chunked"])
def test_step_continues_a_forward_pass(algo):
    """Final states of a forward pass over L tokens, then one step, equal the
    oracle over L + 1 tokens (the decode loop after a prefill)."""
    import ssd_scan_amd as ssd

    L = 300
    full = ssd_synth.random_case(210, 2, L + 1, 4, 64, 64, 2, chunk=128, dtype="bf16",
                                 with_init=True)
    tdt = torch.bfloat16
    d = lambda a, t=tdt: _dev(a, t)
    say(f"prefill + step ({algo})")
    _, fin = ssd.fwd(d(full.x[:, :L]), d(full.dt[:, :L]), d(full.A, torch.float32),
                     d(full.B[:, :L]), d(full.C[:, :L]), d(full.D, torch.float32), None,
                     d(full.initial_states, torch.float32), chunk_size=128, dt_min=full.dt_min,
                     dt_max=full.dt_max, algo=algo, return_final_states=True)
    y = ssd.step(d(full.x[:, L]), d(full.dt[:, L]), d(full.A, torch.float32), d(full.B[:, L]),
                 d(full.C[:, L]), fin, d(full.D, torch.float32), None, dt_min=full.dt_min,
                 dt_max=full.dt_max)
    torch.cuda.synchronize()
    yr, fr = oracle.ssd_ref(full.x, full.dt, full.A, full.B, full.C, full.D, None,
                            full.initial_states, softplus=True, dt_min=full.dt_min,
                            dt_max=full.dt_max)
    assert rel_err(y.float().cpu().numpy(), yr[:, L]) < TOL["bf16"]
    assert rel_err(fin.cpu().numpy(), fr) < TOL["bf16"]


def test_step_with_no_rows_is_a_no_op():
    import ssd_scan_amd as ssd

    z = lambda *s: torch.zeros(*s, device="cuda")
    y = ssd.step(z(0, 2, 64), z(0, 2), -torch.ones(2, device="cuda"), z(0, 1, 16), z(0, 1, 16),
                 z(0, 2, 16, 64))
    torch.cuda.synchronize()
    assert y.shape == (0, 2, 64)
