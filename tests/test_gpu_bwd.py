"""GPU parity of the backward pass (``ssd_bwd``) against the fp64 oracle's
gradients (``oracle.ssd_ref_bwd``), through the C ABI.

Each case draws the workload distributions (ssd_synth) plus seeded upstream
gradients dy and d_final_states, runs the HIP backward and the oracle on the
same values, and compares every gradient with the forward pass's error measure
(max_i |g_i - ref_i| / max(|ref_i|, rms(ref))), with the forward pass's
tolerances: 1e-4 for fp32 storage, 2e-2 for bf16 storage (fp32 accumulation).
"""
import numpy as np
import pytest

import oracle
import ssd_synth
from checkers import rel_err
from parity import record, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BWD_TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "ddt_bias", "dinit")

CASES = [
    dict(name="bf16_b2_L300_H4_P64_N64", seed=301, b=2, L=300, H=4, P=64, N=64, G=1,
         dtype="bf16", init=True, dfin=True),
    dict(name="bf16_b1_L256_H8_P64_N128_G2_Gc8_scaled", seed=302, b=1, L=256, H=8, P=64, N=128,
         G=2, Gc=8, dtype="bf16", scales=True, bias=0.3),
    dict(name="bf16_b1_L200_H2_P128_N128", seed=303, b=1, L=200, H=2, P=128, N=128, G=1,
         dtype="bf16", init=True, dfin=True),
    dict(name="bf16_b1_L130_H2_P64_N256_Gc1", seed=304, b=1, L=130, H=2, P=64, N=256, G=2, Gc=1,
         dtype="bf16", dfin=True),
    dict(name="bf16_b3_L1_H2_P64_N32", seed=305, b=3, L=1, H=2, P=64, N=32, G=1, dtype="bf16",
         init=True, dfin=True),
    dict(name="f32_b2_L100_H4_P64_N16_G4", seed=306, b=2, L=100, H=4, P=64, N=16, G=4,
         dtype="f32", init=True, dfin=True),
    dict(name="f32_b1_L129_H3_P128_N64_scaled_bias", seed=307, b=1, L=129, H=3, P=128, N=64, G=1,
         dtype="f32", scales=True, bias=-0.5, init=True),
    dict(name="f32_b1_L64_H2_P64_N128_noD", seed=308, b=1, L=64, H=2, P=64, N=128, G=1,
         dtype="f32", noD=True),
    dict(name="f32_b1_L333_H2_P64_N32_G1_Gc2", seed=309, b=1, L=333, H=2, P=64, N=32, G=1, Gc=2,
         dtype="f32", init=True, dfin=True),
]


# packed sequences (b = 1), from zero states with no final-state gradient
VARLEN_CASES = [
    dict(name="bf16_packed_H4_P64_N64", seed=331, H=4, P=64, N=64, G=1, dtype="bf16",
         lengths=[128, 0, 64, 1, 300, 5, 142]),
    dict(name="f32_packed_H2_P64_N32_scaled", seed=332, H=2, P=64, N=32, G=1, dtype="f32",
         lengths=[70, 33, 200, 1], scales=True),
    dict(name="bf16_packed_H4_P128_N128_G1_Gc4", seed=333, H=4, P=128, N=128, G=1, Gc=4,
         dtype="bf16", lengths=[500, 12, 64, 0, 37]),
]

# packed sequences with per-sequence initial states and/or final-state
# gradients: empty and one-token sequences, starts on and off the 64-token
# chunk grid, several sequences inside one chunk, sequences over many chunks
VARLEN_STATE_CASES = [
    dict(name="bf16_packed_states_H4_P64_N64", seed=351, H=4, P=64, N=64, G=1, dtype="bf16",
         lengths=[128, 0, 64, 1, 300, 5, 142], init=True, dfin=True),
    dict(name="f32_packed_init_H2_P64_N32_scaled", seed=352, H=2, P=64, N=32, G=1, dtype="f32",
         lengths=[70, 33, 200, 1], scales=True, init=True),
    dict(name="f32_packed_dfinal_H3_P128_N64_bias", seed=353, H=3, P=128, N=64, G=1, dtype="f32",
         lengths=[3, 60, 1, 0, 129], dfin=True, bias=-0.4),
    dict(name="bf16_packed_states_H4_P128_N128_G1_Gc4_scaled", seed=354, H=4, P=128, N=128, G=1,
         Gc=4, dtype="bf16", lengths=[500, 12, 64, 0, 37], init=True, dfin=True, scales=True),
    dict(name="bf16_packed_states_H2_P64_N256_G2_Gc1", seed=355, H=2, P=64, N=256, G=2, Gc=1,
         dtype="bf16", lengths=[90, 40, 17], init=True, dfin=True),
    dict(name="f32_packed_states_H2_P64_N16_many_short", seed=356, H=2, P=64, N=16, G=1,
         dtype="f32", lengths=[1, 2, 3, 0, 5, 8, 13, 21, 34, 55, 1, 1], init=True, dfin=True),
]


def _dev(a, dtype):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype)


def _draw(c):
    inp = ssd_synth.random_case(c["seed"], c["b"], c["L"], c["H"], c["P"], c["N"], c["G"],
                                dtype=c["dtype"], with_init=c.get("init", False),
                                with_D=not c.get("noD", False), Gc=c.get("Gc"))
    if "bias" in c:
        inp.dt_bias = np.full(c["H"], c["bias"], np.float32)
    inp.scales_input = c.get("scales", False)
    dy, dfin = ssd_synth.random_grads(c["seed"] + 1000, inp, with_dfinal=c.get("dfin", False))
    return inp, dy, dfin


def _run(inp, dy, dfin):
    import ssd_scan_amd as ssd

    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    f32 = torch.float32
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens).to("cuda")
    out = ssd.bwd(_dev(inp.x, tdt), _dev(inp.dt, tdt), _dev(inp.A, f32), _dev(inp.B, tdt),
                  _dev(inp.C, tdt), _dev(dy, tdt), _dev(inp.D, f32), _dev(inp.dt_bias, f32),
                  _dev(inp.initial_states, f32), _dev(dfin, f32), cu, softplus=inp.softplus,
                  scales_input=inp.scales_input, dt_min=inp.dt_min, dt_max=inp.dt_max)
    torch.cuda.synchronize()
    return {k: None if out[k] is None else out[k].float().cpu().numpy() for k in NAMES}


def _oracle(inp, dy, dfin):
    return oracle.ssd_ref_bwd(inp.x, inp.dt, inp.A, inp.B, inp.C, dy, inp.D, inp.dt_bias,
                              inp.initial_states, inp.cu_seqlens, dfin, softplus=inp.softplus,
                              scales_input=inp.scales_input, dt_min=inp.dt_min,
                              dt_max=inp.dt_max)


@pytest.mark.parametrize("c", CASES, ids=[c["name"] for c in CASES])
def test_bwd_matches_oracle(c):
    inp, dy, dfin = _draw(c)
    say(f"bwd {c['name']}")
    got = _run(inp, dy, dfin)
    ref = _oracle(inp, dy, dfin)
    tol = BWD_TOL[c["dtype"]]
    errs = {k: rel_err(got[k], ref[k]) for k in NAMES}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{c['name']}: rel err above {tol}: {bad} (all: {errs})"


@pytest.mark.parametrize("c", [c for c in CASES if c["dtype"] == "bf16"],
                         ids=[c["name"] for c in CASES if c["dtype"] == "bf16"])
def test_bwd_walks_match_oracle(c, monkeypatch):
    """Dense bf16 rows take the state walks (S_in and G_end formed by walking
    each stream with the state in registers) when their grid fills the device,
    else the per-chunk state kernels and the two scans; SSD_BWD_WALK=1 makes
    these small cases take the walks, which must agree with the oracle as
    well."""
    monkeypatch.setenv("SSD_BWD_WALK", "1")
    inp, dy, dfin = _draw(c)
    say(f"bwd (state walks) {c['name']}")
    got = _run(inp, dy, dfin)
    ref = _oracle(inp, dy, dfin)
    tol = BWD_TOL[c["dtype"]]
    errs = {k: rel_err(got[k], ref[k]) for k in NAMES}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{c['name']}: rel err above {tol}: {bad} (all: {errs})"


# heads of one B / C group walked by one workgroup (dB and dC summed over the
# block in place), forced at sizes the oracle finishes in seconds
HEAD_BLOCK_CASES = [
    dict(name="bf16_b2_L300_H8_P64_N128_blk8", seed=361, b=2, L=300, H=8, P=64, N=128, G=1,
         dtype="bf16", init=True, dfin=True),
    dict(name="bf16_b1_L200_H12_P64_N64_Gc3_blk4_scaled", seed=362, b=1, L=200, H=12, P=64, N=64,
         G=1, Gc=3, dtype="bf16", scales=True, bias=0.2, init=True),
    dict(name="bf16_b1_L130_H4_P128_N128_G2_blk2", seed=363, b=1, L=130, H=4, P=128, N=128, G=2,
         dtype="bf16", dfin=True),
    dict(name="f32_b2_L100_H8_P64_N32_G2_blk4", seed=364, b=2, L=100, H=8, P=64, N=32, G=2,
         dtype="f32", init=True, dfin=True),
]


@pytest.mark.parametrize("c", HEAD_BLOCK_CASES, ids=[c["name"] for c in HEAD_BLOCK_CASES])
@pytest.mark.parametrize("walk", ["walk", "nowalk"])
def test_bwd_head_blocks_match_oracle(c, walk, monkeypatch):
    """SSD_BWD_HEAD_BLOCK=8 makes every workgroup of the chunk kernel take
    the largest block of 8, 4, 2 heads dividing the group sizes (the full-size
    layer takes blocks of 8 by itself)."""
    monkeypatch.setenv("SSD_BWD_HEAD_BLOCK", "8")
    monkeypatch.setenv("SSD_BWD_WALK" if walk == "walk" else "SSD_BWD_NO_WALK", "1")
    inp, dy, dfin = _draw(c)
    say(f"bwd head blocks ({walk}) {c['name']}")
    got = _run(inp, dy, dfin)
    ref = _oracle(inp, dy, dfin)
    tol = BWD_TOL[c["dtype"]]
    errs = {k: rel_err(got[k], ref[k]) for k in NAMES}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{c['name']}: rel err above {tol}: {bad} (all: {errs})"


@pytest.mark.parametrize("c", VARLEN_CASES, ids=[c["name"] for c in VARLEN_CASES])
def test_bwd_packed_sequences_match_oracle(c):
    """Packed sequences (section 8.3): nothing flows between sequences, in
    either direction; empty and one-token sequences, sequences that start on a
    chunk boundary and several sequences inside one chunk."""
    L = sum(c["lengths"])
    inp = ssd_synth.random_case(c["seed"], 1, L, c["H"], c["P"], c["N"], c["G"],
                                dtype=c["dtype"], lengths=c["lengths"], Gc=c.get("Gc"))
    inp.scales_input = c.get("scales", False)
    dy, _ = ssd_synth.random_grads(c["seed"] + 1000, inp, with_dfinal=False)
    say(f"bwd packed {c['name']}")
    got = _run(inp, dy, None)
    ref = _oracle(inp, dy, None)
    assert got["dinit"].shape == (len(c["lengths"]), c["H"], c["N"], c["P"])
    tol = BWD_TOL[c["dtype"]]
    errs = {k: rel_err(got[k], ref[k]) for k in NAMES}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{c['name']}: rel err above {tol}: {bad} (all: {errs})"


@pytest.mark.parametrize("c", VARLEN_STATE_CASES, ids=[c["name"] for c in VARLEN_STATE_CASES])
def test_bwd_packed_sequences_with_states_match_oracle(c):
    """Packed sequences with their own initial states and final-state
    gradients (section 8.3): each sequence's first state decays its initial
    state, the gradient of each final state enters at that sequence's last
    token, and the initial-state gradient is taken per sequence."""
    L = sum(c["lengths"])
    inp = ssd_synth.random_case(c["seed"], 1, L, c["H"], c["P"], c["N"], c["G"],
                                dtype=c["dtype"], lengths=c["lengths"], Gc=c.get("Gc"),
                                with_init=c.get("init", False))
    if "bias" in c:
        inp.dt_bias = np.full(c["H"], c["bias"], np.float32)
    inp.scales_input = c.get("scales", False)
    dy, dfin = ssd_synth.random_grads(c["seed"] + 1000, inp, with_dfinal=c.get("dfin", False))
    say(f"bwd packed with states {c['name']}")
    got = _run(inp, dy, dfin)
    ref = _oracle(inp, dy, dfin)
    tol = BWD_TOL[c["dtype"]]
    errs = {k: rel_err(got[k], ref[k]) for k in NAMES}
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{c['name']}: rel err above {tol}: {bad} (all: {errs})"


def test_bwd_packed_empty_sequences_pass_the_final_gradients_through():
    """Packed sequences that are all empty: each initial-state gradient is that
    sequence's final-state gradient, and the per-head sums are zero."""
    import ssd_scan_amd as ssd

    inp = ssd_synth.random_case(357, 1, 0, 2, 64, 16, 1, dtype="f32", lengths=[0, 0, 0],
                                with_init=True)
    _, dfin = ssd_synth.random_grads(358, inp)
    f32 = torch.float32
    cu = torch.from_numpy(inp.cu_seqlens).to("cuda")
    out = ssd.bwd(_dev(inp.x, f32), _dev(inp.dt, f32), _dev(inp.A, f32), _dev(inp.B, f32),
                  _dev(inp.C, f32), _dev(inp.x, f32), _dev(inp.D, f32), None,
                  _dev(inp.initial_states, f32), _dev(dfin, f32), cu)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["dinit"].cpu().numpy(), dfin)
    for k in ("dA", "dD", "ddt_bias"):
        np.testing.assert_array_equal(out[k].cpu().numpy(), np.zeros(2, np.float32))


def test_bwd_empty_sequence_passes_the_final_gradient_through():
    import ssd_scan_amd as ssd

    inp = ssd_synth.random_case(311, 2, 0, 2, 64, 16, 1, dtype="bf16", with_init=True)
    _, dfin = ssd_synth.random_grads(312, inp)
    out = ssd.bwd(_dev(inp.x, torch.bfloat16), _dev(inp.dt, torch.bfloat16),
                  _dev(inp.A, torch.float32), _dev(inp.B, torch.bfloat16),
                  _dev(inp.C, torch.bfloat16), _dev(inp.x, torch.bfloat16),
                  _dev(inp.D, torch.float32), None, _dev(inp.initial_states, torch.float32),
                  _dev(dfin, torch.float32))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out["dinit"].cpu().numpy(), dfin)
    for k in ("dA", "dD", "ddt_bias"):
        np.testing.assert_array_equal(out[k].cpu().numpy(), np.zeros(2, np.float32))


def test_bwd_full_size_every_head():
    """The 2.7B-shaped layer (b4 L4096 H80 P64 N128 G1, bf16) in the launch
    configuration the benchmark times, every gradient over every head against
    the oracle, including dB and dC, which sum over all 80 heads sharing the
    B/C group; the observed errors are recorded."""
    inp = ssd_synth.make("mamba2_2p7b")
    b, L, H, P = inp.x.shape
    rng = np.random.default_rng(321)
    init = rng.standard_normal((b, H, inp.B.shape[3], P), dtype=np.float32)
    inp.initial_states = init
    dy, dfin = ssd_synth.random_grads(322, inp)
    say("bwd full size b4 L4096 H80 P64 N128 (every head)")
    got = _run(inp, dy, dfin)
    ref = _oracle(inp, dy, dfin)
    errs = {k: rel_err(got[k], ref[k]) for k in NAMES}
    record("bwd mamba2_2p7b", **errs)
    bad = {k: v for k, v in errs.items() if not v <= BWD_TOL["bf16"]}
    assert not bad, f"rel err above {BWD_TOL['bf16']}: {bad} (all: {errs})"


def test_bwd_rejects_unsupported_shapes():
    import ctypes

    import ssd_scan_amd as ssd

    lib = ssd.library()
    p = ssd.make_problem(1, 128, 2, 64, 256, 1, 64, bf16=False)
    assert lib.ssd_bwd_workspace_size(ctypes.byref(p)) == 0  # fp32 with N P > 8192
    p = ssd.make_problem(1, 128, 2, 128, 256, 1, 64, bf16=True)
    assert lib.ssd_bwd_workspace_size(ctypes.byref(p)) == 0  # bf16 with N P > 16384
    p = ssd.make_problem(1, 128, 2, 64, 64, 1, 64, bf16=True, nseqs=2)
    assert lib.ssd_bwd_workspace_size(ctypes.byref(p)) > 0  # packed sequences


def test_autograd_function_matches_oracle_gradients():
    """ssd_scan_amd.ssd_scan under torch.autograd: the loss sum(dy y) +
    sum(dfin final) gives the oracle's gradients for every input."""
    import ssd_scan_amd as ssd

    c = dict(seed=341, b=2, L=150, H=4, P=64, N=64, G=2, dtype="bf16", init=True, dfin=True)
    inp, dy, dfin = _draw(c)
    inp.dt_bias = np.full(c["H"], 0.2, np.float32)
    tdt, f32 = torch.bfloat16, torch.float32
    leaf = lambda a, d: _dev(a, d).requires_grad_(True)  # noqa: E731
    x, dt, B, C = (leaf(a, tdt) for a in (inp.x, inp.dt, inp.B, inp.C))
    A, D, bias, init = (leaf(a, f32) for a in (inp.A, inp.D, inp.dt_bias, inp.initial_states))
    say("autograd ssd_scan")
    y, fin = ssd.ssd_scan(x, dt, A, B, C, D, bias, init, dt_min=inp.dt_min, dt_max=inp.dt_max)
    loss = (y.float() * _dev(dy, f32)).sum() + (fin * _dev(dfin, f32)).sum()
    grads = torch.autograd.grad(loss, [x, dt, A, B, C, D, bias, init])
    ref = _oracle(inp, dy, dfin)
    for name, gv in zip(("dx", "ddt", "dA", "dB", "dC", "dD", "ddt_bias", "dinit"), grads):
        err = rel_err(gv.float().cpu().numpy(), ref[name])
        assert err <= BWD_TOL["bf16"], f"{name}: rel err {err:.3e}"


def test_autograd_packed_sequences_with_states():
    """ssd_scan with packed sequences and per-sequence initial states under
    autograd: (y, final_states) per sequence, and the oracle's gradients for
    every input."""
    import ssd_scan_amd as ssd

    lengths = [40, 0, 100, 1, 59]
    inp = ssd_synth.random_case(361, 1, sum(lengths), 4, 64, 32, 2, dtype="bf16",
                                lengths=lengths, with_init=True)
    inp.dt_bias = np.full(4, 0.1, np.float32)
    dy, dfin = ssd_synth.random_grads(362, inp)
    tdt, f32 = torch.bfloat16, torch.float32
    leaf = lambda a, d: _dev(a, d).requires_grad_(True)  # noqa: E731
    x, dt, B, C = (leaf(a, tdt) for a in (inp.x, inp.dt, inp.B, inp.C))
    A, D, bias, init = (leaf(a, f32) for a in (inp.A, inp.D, inp.dt_bias, inp.initial_states))
    cu = torch.from_numpy(inp.cu_seqlens).to("cuda")
    say("autograd ssd_scan packed with states")
    y, fin = ssd.ssd_scan(x, dt, A, B, C, D, bias, init, cu, dt_min=inp.dt_min,
                          dt_max=inp.dt_max)
    assert fin.shape == (len(lengths), 4, 32, 64)
    loss = (y.float() * _dev(dy, f32)).sum() + (fin * _dev(dfin, f32)).sum()
    grads = torch.autograd.grad(loss, [x, dt, A, B, C, D, bias, init])
    ref = _oracle(inp, dy, dfin)
    for name, gv in zip(("dx", "ddt", "dA", "dB", "dC", "dD", "ddt_bias", "dinit"), grads):
        err = rel_err(gv.float().cpu().numpy(), ref[name])
        assert err <= BWD_TOL["bf16"], f"{name}: rel err {err:.3e}"


@pytest.mark.parametrize("walk", ["1", "0", "packed"], ids=["walks", "chunk_states", "packed_states"])
def test_bwd_deterministic_run_to_run(walk, monkeypatch):
    """Two runs of the backward pass give the same bits: dense rows with the
    state walks and with the per-chunk state kernels and scans, and packed
    sequences with per-sequence states and final-state gradients (every sum has
    a fixed order: head blocks in place, group and head sums by fixed trees,
    the per-sequence terms' token sums by butterflies instead of atomics)."""
    if walk == "packed":
        c = dict(seed=392, H=4, P=128, N=128, G=1, Gc=4, dtype="bf16",
                 lengths=[500, 12, 64, 0, 37])
        inp = ssd_synth.random_case(c["seed"], 1, sum(c["lengths"]), c["H"], c["P"], c["N"],
                                    c["G"], dtype=c["dtype"], lengths=c["lengths"], Gc=c["Gc"],
                                    with_init=True)
        inp.scales_input = True
        dy, dfin = ssd_synth.random_grads(c["seed"] + 1000, inp, with_dfinal=True)
    else:
        monkeypatch.setenv("SSD_BWD_WALK" if walk == "1" else "SSD_BWD_NO_WALK", "1")
        c = dict(seed=391, b=2, L=1000, H=8, P=64, N=128, G=2, dtype="bf16", init=True, dfin=True)
        inp, dy, dfin = _draw(c)
    say(f"bwd determinism {walk}")
    g1 = _run(inp, dy, dfin)
    g2 = _run(inp, dy, dfin)
    for k in NAMES:
        assert np.array_equal(g1[k], g2[k]), k
