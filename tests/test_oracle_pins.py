"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  None of them re-types the oracle's loop: each
compares it with a different formulation or a closed form ("Transformers are
SSMs": section 3.1/3.3 matrix form, section 3.2.2 and appendix B.1 scalar
recurrence special cases, section 4.2.1 causal mask = cumulative sum, section 6
block decomposition, appendix B.3.3 chunk size 1, section 8.2 state hand-off,
section 8.3 variable length, section 7.1 shared B/C heads).
"""
import json
import os

import numpy as np
import pytest

import oracle
import ssd_synth
from checkers import chunked_form, dt_effective, quadratic_form, rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def run(inp, lib=None, **kw):
    args = dict(softplus=inp.softplus, scales_input=inp.scales_input, dt_min=inp.dt_min,
                dt_max=inp.dt_max)
    args.update(kw)
    return oracle.ssd_ref(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.dt_bias,
                          inp.initial_states, inp.cu_seqlens, lib=lib, **args)


def check_kwargs(inp):
    return dict(D=inp.D, dt_bias=inp.dt_bias, init=inp.initial_states, cu=inp.cu_seqlens,
                softplus=inp.softplus, scales_input=inp.scales_input, dt_min=inp.dt_min,
                dt_max=inp.dt_max)


# ---------------------------------------------------------------- worked examples
def test_golden_worked_examples(oracle_lib):
    spec = json.load(open(GOLDEN))
    for case in spec["cases"]:
        sh = case["shape"]
        b, L, H, P, N, G = (sh[k] for k in ("batch", "seqlen", "H", "P", "N", "G"))
        x = np.array(case["x"], np.float32).reshape(b, L, H, P)
        dt = np.array(case["dt"], np.float32).reshape(b, L, H)
        A = np.array([case["A"]], np.float32)
        B = np.array(case["B"], np.float32).reshape(b, L, G, N)
        C = np.array(case["C"], np.float32).reshape(b, L, G, N)
        D = np.array([case["D"]], np.float32)
        cu = None if case["cu_seqlens"] is None else np.array(case["cu_seqlens"], np.int32)
        nseq = b if cu is None else len(cu) - 1
        init = None
        if case["initial_state"] is not None:
            init = np.array(case["initial_state"], np.float32).reshape(nseq, H, N, P)
        y, fin = oracle.ssd_ref(x, dt, A, B, C, D, None, init, cu, softplus=False, lib=oracle_lib)
        np.testing.assert_allclose(y.reshape(-1), case["y"], rtol=spec["tolerance_rel"], atol=1e-12)
        np.testing.assert_allclose(fin.reshape(nseq, -1), np.array(case["final_states"]),
                                   rtol=spec["tolerance_rel"], atol=1e-12)


# ---------------------------------------------------------------- brute force (quadratic form)
QUAD_CASES = [
    dict(seed=1, batch=2, seqlen=37, H=3, P=5, N=4, G=1),
    dict(seed=2, batch=1, seqlen=64, H=4, P=8, N=6, G=2, with_init=True),
    dict(seed=3, batch=3, seqlen=17, H=2, P=3, N=7, G=2, with_init=True),
    dict(seed=4, batch=1, seqlen=50, H=4, P=4, N=3, G=4, lengths=[7, 0, 20, 1, 22], with_init=True),
    dict(seed=5, batch=1, seqlen=40, H=2, P=4, N=5, G=1, lengths=[13, 27]),
]


@pytest.mark.parametrize("case", QUAD_CASES)
@pytest.mark.parametrize("scales_input", [False, True])
def test_quadratic_form(oracle_lib, case, scales_input):
    inp = ssd_synth.random_case(**case)
    inp.scales_input = scales_input
    inp.dt_bias = np.linspace(-0.5, 0.5, inp.x.shape[2]).astype(np.float32)
    # a wider clamp so the decays spread out
    inp.dt_min, inp.dt_max = 1e-3, 0.5
    y, fin = run(inp, oracle_lib)
    yq, fq = quadratic_form(inp.x, inp.dt, inp.A, inp.B, inp.C, **check_kwargs(inp))
    assert rel_err(y, yq) < 1e-12
    assert rel_err(fin, fq) < 1e-12


def test_quadratic_form_strong_decay_and_growth(oracle_lib):
    """Decays spanning many orders of magnitude, and A > 0 (growth) on a short sequence."""
    inp = ssd_synth.random_case(11, 1, 24, 3, 4, 3, 1)
    inp.A = np.array([-16.0, -0.05, 0.7], np.float32)
    inp.dt_min, inp.dt_max = 0.0, 2.0
    y, fin = run(inp, oracle_lib)
    yq, fq = quadratic_form(inp.x, inp.dt, inp.A, inp.B, inp.C, **check_kwargs(inp))
    assert rel_err(y, yq) < 1e-12
    assert rel_err(fin, fq) < 1e-12


# ---------------------------------------------------------------- special cases of the scan
def test_a_equals_one_is_causal_linear_attention(oracle_lib):
    """A = 0 => a_t = 1: the mask multiplication is a cumulative sum (section 4.2.1, B.1)."""
    inp = ssd_synth.random_case(21, 2, 33, 3, 4, 5, 1, with_init=True)
    inp.A = np.zeros(3, np.float32)
    y, fin = run(inp, oracle_lib)
    x = inp.x.astype(np.float64)
    B = inp.B.astype(np.float64)[:, :, 0]
    C = inp.C.astype(np.float64)[:, :, 0]
    outer = B[:, :, None, :, None] * x[:, :, :, None, :]  # (b, L, H, N, P)
    S = np.cumsum(outer, axis=1) + inp.initial_states.astype(np.float64)[:, None]
    expect = np.einsum("bln,blhnp->blhp", C, S) + inp.D[None, None, :, None] * x
    assert rel_err(y, expect) < 1e-12
    assert rel_err(fin, S[:, -1]) < 1e-12


def test_a_equals_zero_keeps_only_the_current_token(oracle_lib):
    """A = -1e6, dt >= 1e-3 => a_t underflows to exactly 0: y_t = (C_t . B_t) x_t + D x_t."""
    inp = ssd_synth.random_case(22, 2, 19, 2, 3, 4, 2, with_init=True)
    inp.A = np.full(2, -1e6, np.float32)
    y, fin = run(inp, oracle_lib)
    x = inp.x.astype(np.float64)
    cb = np.einsum("blgn,blgn->blg", inp.C.astype(np.float64), inp.B.astype(np.float64))
    heads_g = np.arange(2) // 1  # G == H == 2
    expect = cb[:, :, heads_g, None] * x + inp.D[None, None, :, None] * x
    assert rel_err(y, expect) < 1e-13
    last = inp.B.astype(np.float64)[:, -1, heads_g, :, None] * x[:, -1, :, None, :]
    assert rel_err(fin, last) < 1e-13


def test_zero_input_is_cumulative_product_of_the_initial_state(oracle_lib):
    """x = 0 => y_t = C_t^T (prod_{k<=t} a_k) S_init: the cumprod case (appendix B.1)."""
    inp = ssd_synth.random_case(23, 1, 45, 3, 4, 6, 3, with_init=True)
    inp.x[:] = 0
    y, fin = run(inp, oracle_lib)
    a = np.exp(dt_effective(inp.dt, None, True, inp.dt_min, inp.dt_max) * inp.A[None, None, :])
    pa = np.cumprod(a, axis=1)  # (b, L, H)
    init = inp.initial_states.astype(np.float64)
    expect = np.einsum("blhn,bhnp->blhp", inp.C.astype(np.float64), init) * pa[..., None]
    assert rel_err(y, expect) < 1e-12
    assert rel_err(fin, init * pa[:, -1, :, None, None]) < 1e-12


def test_zero_B_or_C_leaves_the_skip_term(oracle_lib):
    for which in ("B", "C"):
        inp = ssd_synth.random_case(24, 2, 21, 3, 5, 4, 1)
        getattr(inp, which)[:] = 0
        y, _ = run(inp, oracle_lib)
        expect = inp.D[None, None, :, None].astype(np.float64) * inp.x.astype(np.float64)
        assert np.array_equal(y, expect)


def test_without_D_there_is_no_skip(oracle_lib):
    inp = ssd_synth.random_case(25, 1, 16, 2, 3, 4, 1, with_D=False)
    inp.B[:] = 0
    y, _ = run(inp, oracle_lib)
    assert np.all(y == 0)


# ---------------------------------------------------------------- structure
def test_linearity_in_x_and_initial_state(oracle_lib):
    """y(a x1 + b x2, a i1 + b i2) = a y(x1, i1) + b y(x2, i2), on inputs whose
    combination is exact in float32 (multiples of 1/64, |value| < 8)."""
    i1 = ssd_synth.random_case(31, 2, 29, 3, 4, 5, 1, with_init=True, with_D=False)
    i2 = ssd_synth.random_case(32, 2, 29, 3, 4, 5, 1, with_init=True, with_D=False)
    q = lambda v: (np.round(np.clip(v, -3, 3) * 64) / 64).astype(np.float32)
    i1.x, i2.x = q(i1.x), q(i2.x)
    i1.initial_states, i2.initial_states = q(i1.initial_states), q(i2.initial_states)
    i2.dt, i2.A, i2.B, i2.C = i1.dt, i1.A, i1.B, i1.C
    y1, f1 = run(i1, oracle_lib)
    y2, f2 = run(i2, oracle_lib)
    for al, be in ((1.0, -2.0), (0.5, 0.25), (-1.0, 1.0)):
        i3 = ssd_synth.random_case(31, 2, 29, 3, 4, 5, 1, with_init=True, with_D=False)
        i3.dt, i3.A, i3.B, i3.C = i1.dt, i1.A, i1.B, i1.C
        i3.x = (np.float32(al) * i1.x + np.float32(be) * i2.x).astype(np.float32)
        i3.initial_states = (np.float32(al) * i1.initial_states
                             + np.float32(be) * i2.initial_states).astype(np.float32)
        assert np.array_equal(i3.x.astype(np.float64), al * i1.x.astype(np.float64)
                              + be * i2.x.astype(np.float64))
        y3, f3 = run(i3, oracle_lib)
        assert rel_err(y3, al * y1 + be * y2) < 1e-12
        assert rel_err(f3, al * f1 + be * f2) < 1e-12


@pytest.mark.parametrize("Q", [1, 3, 16, 64, 1000])
def test_block_decomposition_matches_recurrence(oracle_lib, Q):
    """Chunked evaluation (section 6) equals the recurrence for any chunk length."""
    for case in (dict(seed=41, batch=2, seqlen=100, H=3, P=4, N=5, G=1, with_init=True),
                 dict(seed=42, batch=1, seqlen=90, H=4, P=3, N=4, G=2,
                      lengths=[30, 0, 45, 15], with_init=True)):
        inp = ssd_synth.random_case(**case)
        inp.dt_max = 0.5
        y, fin = run(inp, oracle_lib)
        yc, fc = chunked_form(inp.x, inp.dt, inp.A, inp.B, inp.C, Q, **check_kwargs(inp))
        assert rel_err(y, yc) < 1e-11
        assert rel_err(fin, fc) < 1e-11


def test_varlen_equals_separate_runs(oracle_lib):
    lengths = [11, 0, 25, 1, 40]
    inp = ssd_synth.random_case(51, 1, sum(lengths), 4, 3, 5, 2, lengths=lengths, with_init=True)
    y, fin = run(inp, oracle_lib)
    cu = inp.cu_seqlens
    for s in range(len(lengths)):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        ys, fs = oracle.ssd_ref(inp.x[:, t0:t1], inp.dt[:, t0:t1], inp.A, inp.B[:, t0:t1],
                                inp.C[:, t0:t1], inp.D, None, inp.initial_states[s:s + 1], None,
                                softplus=True, dt_min=inp.dt_min, dt_max=inp.dt_max, lib=oracle_lib)
        assert np.array_equal(y[:, t0:t1], ys)
        assert np.array_equal(fin[s:s + 1], fs)


def test_varlen_is_recurrence_with_zero_decay_at_starts(oracle_lib):
    """Section 8.3: one long sequence with A_t = 0 (no carry) at every start."""
    lengths = [9, 14, 1, 20]
    inp = ssd_synth.random_case(52, 1, sum(lengths), 2, 3, 4, 1, lengths=lengths)
    y, fin = run(inp, oracle_lib)
    # the packed stream against the matrix form with no decay path across a start
    yq, fq = quadratic_form(inp.x, inp.dt, inp.A, inp.B, inp.C, **check_kwargs(inp))
    assert rel_err(y, yq) < 1e-12
    # and the first token of each sequence sees only itself
    cu = inp.cu_seqlens
    for s in range(len(lengths)):
        t = int(cu[s])
        for h in range(2):
            cb = float(inp.C[0, t, 0].astype(np.float64) @ inp.B[0, t, 0].astype(np.float64))
            xt = inp.x[0, t, h].astype(np.float64)
            expect = cb * xt + float(inp.D[h]) * xt
            np.testing.assert_allclose(y[0, t, h], expect, rtol=1e-13, atol=1e-15)


def test_state_handoff_split_and_carry(oracle_lib):
    """Section 8.2: run [0, t0) then [t0, T) from the handed-over state == one run."""
    inp = ssd_synth.random_case(61, 2, 70, 3, 4, 5, 1, with_init=True)
    y, fin = run(inp, oracle_lib)
    for t0 in (1, 31, 69):
        ya, fa = oracle.ssd_ref(inp.x[:, :t0], inp.dt[:, :t0], inp.A, inp.B[:, :t0], inp.C[:, :t0],
                                inp.D, None, inp.initial_states, None, softplus=True,
                                dt_min=inp.dt_min, dt_max=inp.dt_max, lib=oracle_lib)
        # the handed-over state is fp64; the oracle takes fp32 initial states, so
        # compare the second half against the quadratic form fed with the fp64 state
        yb, fb = quadratic_form(inp.x[:, t0:], inp.dt[:, t0:], inp.A, inp.B[:, t0:],
                                inp.C[:, t0:], D=inp.D, init=fa, softplus=True,
                                dt_min=inp.dt_min, dt_max=inp.dt_max)
        assert np.array_equal(ya, y[:, :t0])
        assert rel_err(yb, y[:, t0:]) < 1e-12
        assert rel_err(fb, fin) < 1e-12


def test_group_broadcast_equals_replicated_heads(oracle_lib):
    """Section 7.1/7.2: G shared B/C heads == every x head with its own copy."""
    inp = ssd_synth.random_case(71, 2, 23, 6, 3, 4, 2, with_init=True)
    y, fin = run(inp, oracle_lib)
    rep = np.repeat(np.arange(2), 3)  # head h -> group h // 3
    yr, fr = oracle.ssd_ref(inp.x, inp.dt, inp.A, np.ascontiguousarray(inp.B[:, :, rep]),
                            np.ascontiguousarray(inp.C[:, :, rep]), inp.D, None,
                            inp.initial_states, None, softplus=True, dt_min=inp.dt_min,
                            dt_max=inp.dt_max, lib=oracle_lib)
    assert np.array_equal(y, yr) and np.array_equal(fin, fr)


@pytest.mark.parametrize("G,Gc", [(1, 6), (6, 1), (2, 3), (3, 2)])
def test_separate_B_and_C_groups_equal_replicated_heads(oracle_lib, G, Gc):
    """Section 7.2 head patterns: B heads shared by H/G and C heads by H/Gc x
    heads (G = 1, Gc = H: multi-contract; G = H, Gc = 1: multi-expand) == every
    x head with its own copies of its B and C heads."""
    lib = oracle_lib
    H = 6
    inp = ssd_synth.random_case(72, 2, 19, H, 3, 4, G, with_init=True, Gc=Gc)
    y, fin = run(inp, lib)
    rb = np.arange(H) // (H // G)
    rc = np.arange(H) // (H // Gc)
    yr, fr = oracle.ssd_ref(inp.x, inp.dt, inp.A, np.ascontiguousarray(inp.B[:, :, rb]),
                            np.ascontiguousarray(inp.C[:, :, rc]), inp.D, None,
                            inp.initial_states, None, softplus=True, dt_min=inp.dt_min,
                            dt_max=inp.dt_max, lib=lib)
    assert np.array_equal(y, yr) and np.array_equal(fin, fr)


def test_input_scaling_flag_is_scaling_x_by_dt(oracle_lib):
    inp = ssd_synth.random_case(81, 1, 30, 2, 3, 4, 1)
    y1, f1 = run(inp, oracle_lib, scales_input=True)
    dte = dt_effective(inp.dt, None, True, inp.dt_min, inp.dt_max)
    x = inp.x.astype(np.float64)
    xs = x * dte[..., None]
    # y_flag(x) - D x == y(dt' x) - D dt' x; with D = 0 both sides are the SSM part
    inp.D = None
    y0, _ = run(inp, oracle_lib, scales_input=True)
    # the oracle takes fp32 inputs, so evaluate the right side with the quadratic form in fp64
    yq, fq = quadratic_form(xs, inp.dt, inp.A, inp.B, inp.C, softplus=True, dt_min=inp.dt_min,
                            dt_max=inp.dt_max)
    assert rel_err(y0, yq) < 1e-12
    assert rel_err(f1, fq) < 1e-12


# ---------------------------------------------------------------- dt preprocessing
def test_dt_preprocessing_softplus_bias_and_clamp(oracle_lib):
    """One token from a unit state: y_0 = exp(dt' A) exactly exposes dt'."""
    raw = np.array([-30.0, -8.0, -4.6, -1.0, 0.0, 0.3, 2.0, 25.0], np.float32)
    T = len(raw)
    for softplus in (False, True):
        for bias, lo, hi in ((0.0, 0.0, np.inf), (0.25, 1e-3, 0.1), (-0.5, 0.05, 3.0)):
            # T independent sequences of one token each (batch T), head count 1, N = P = 1
            x = np.zeros((T, 1, 1, 1), np.float32)
            dt = raw.reshape(T, 1, 1)
            A = np.array([-0.37], np.float32)
            B = np.zeros((T, 1, 1, 1), np.float32)
            C = np.ones((T, 1, 1, 1), np.float32)
            init = np.ones((T, 1, 1, 1), np.float32)
            y, _ = oracle.ssd_ref(x, dt, A, B, C, None, np.array([bias], np.float32), init,
                                  softplus=softplus, dt_min=lo, dt_max=hi, lib=oracle_lib)
            expect_dt = dt_effective(raw.astype(np.float64), np.float32(bias), softplus, lo, hi)
            got_dt = np.log(y.reshape(T)) / float(A[0])
            np.testing.assert_allclose(got_dt, expect_dt, rtol=1e-12, atol=1e-14)


def test_pairs_subset_matches_full_run(oracle_lib):
    inp = ssd_synth.random_case(91, 3, 40, 4, 3, 5, 2, with_init=True)
    y, fin = run(inp, oracle_lib)
    pairs = [(0, 3), (2, 0), (1, 1)]
    ys, fs = run(inp, oracle_lib, pairs=pairs)
    for s, h in pairs:
        assert np.array_equal(ys[s, :, h], y[s, :, h])
        assert np.array_equal(fs[s, h], fin[s, h])
    assert np.isnan(ys[0, :, 0]).all()


def test_synthetic_recipe_distributions():
    """The generator draws what its header says (checked on the tiny fp32 workload)."""
    inp = ssd_synth.make("tiny_f32")
    assert inp.x.shape == (1, 256, 2, 64) and inp.B.shape == (1, 256, 1, 16)
    assert np.all((inp.A <= -1.0) & (inp.A >= -16.0))
    assert abs(float(inp.B.std()) - 0.25) < 0.02
    d = dt_effective(inp.dt, None, True, inp.dt_min, inp.dt_max)
    assert d.min() >= 1e-3 and d.max() <= 0.1
    bf = ssd_synth.round_to_bf16(np.array([1.0, 1.00390625, 1.005859375, -3.14159], np.float32))
    assert np.array_equal(bf, np.array([1.0, 1.0, 1.0078125, -3.140625], np.float32))


# ---------------------------------------------------------------- single-token step
def _step_case(seed, b=3, H=4, P=8, N=6, G=2):
    rng = np.random.default_rng(seed)
    f = lambda *sh: rng.standard_normal(sh).astype(np.float32)
    return dict(x=f(b, H, P), dt=(0.05 + 0.1 * rng.random((b, H))).astype(np.float32),
                B=f(b, G, N), C=f(b, G, N), D=f(H), S=f(b, H, N, P), G=G)


def _group(M, H, G):
    """(b, G, N) -> (b, H, N): the group each head reads (section 7.1)."""
    return np.repeat(M.astype(np.float64), H // G, axis=1)


def test_step_decay_zero_keeps_only_the_token(oracle_lib):
    """a = 0: the new state is B x^T alone and y = (C . B) x + D x."""
    c = _step_case(1)
    b, H, P = c["x"].shape
    A = np.full(H, -1e6, np.float32)
    y, S = oracle.ssd_ref_step(c["x"], c["dt"], A, c["B"], c["C"], c["D"], None, c["S"],
                               lib=oracle_lib)
    Bh, Ch = _group(c["B"], H, c["G"]), _group(c["C"], H, c["G"])
    x = c["x"].astype(np.float64)
    np.testing.assert_allclose(S, Bh[..., :, None] * x[..., None, :], rtol=1e-12, atol=1e-300)
    cb = np.sum(Ch * Bh, axis=-1)
    np.testing.assert_allclose(y, (cb[..., None] + c["D"][None, :, None]) * x, rtol=1e-12,
                               atol=1e-12)


def test_step_decay_one_adds_the_outer_product(oracle_lib):
    """a = 1 (A = 0): S' = S + B x^T, and y reads S' through C."""
    c = _step_case(2)
    b, H, P = c["x"].shape
    A = np.zeros(H, np.float32)
    y, S = oracle.ssd_ref_step(c["x"], c["dt"], A, c["B"], c["C"], None, None, c["S"],
                               lib=oracle_lib)
    Bh, Ch = _group(c["B"], H, c["G"]), _group(c["C"], H, c["G"])
    Sn = c["S"].astype(np.float64) + Bh[..., :, None] * c["x"].astype(np.float64)[..., None, :]
    np.testing.assert_allclose(S, Sn, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y, np.einsum("bhn,bhnp->bhp", Ch, Sn), rtol=1e-12, atol=1e-12)


def test_step_zero_input_decays_the_state(oracle_lib):
    """x = 0: S' = exp(dt A) S and y = exp(dt A) S^T C."""
    c = _step_case(3)
    b, H, P = c["x"].shape
    A = -np.linspace(0.5, 3.0, H).astype(np.float32)
    x0 = np.zeros_like(c["x"])
    y, S = oracle.ssd_ref_step(x0, c["dt"], A, c["B"], c["C"], c["D"], None, c["S"],
                               lib=oracle_lib)
    a = np.exp(c["dt"].astype(np.float64) * A.astype(np.float64))
    Sn = a[..., None, None] * c["S"].astype(np.float64)
    np.testing.assert_allclose(S, Sn, rtol=1e-12)
    Ch = _group(c["C"], H, c["G"])
    np.testing.assert_allclose(y, np.einsum("bhn,bhnp->bhp", Ch, Sn), rtol=1e-12, atol=1e-12)


def test_steps_chain_to_the_sequence(oracle_lib):
    """T steps from an initial state reproduce a T-token run (outputs and final
    state): the step is the recurrence's token update, with softplus, a bias,
    the clamp and the input-scaling flag all on."""
    inp = ssd_synth.random_case(4, 2, 9, 3, 8, 5, 3, chunk=4, dtype="f32", with_init=True)
    bias = np.linspace(-0.5, 0.5, 3).astype(np.float32)
    kw = dict(softplus=True, scales_input=True, dt_min=0.02, dt_max=0.05)
    y, fin = oracle.ssd_ref(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, bias,
                            inp.initial_states, lib=oracle_lib, **kw)
    S = inp.initial_states
    for t in range(inp.x.shape[1]):
        yt, S64 = oracle.ssd_ref_step(inp.x[:, t], inp.dt[:, t], inp.A, inp.B[:, t], inp.C[:, t],
                                      inp.D, bias, S, lib=oracle_lib, **kw)
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-5, atol=1e-6)
        S = S64.astype(np.float32)
    np.testing.assert_allclose(S, fin, rtol=1e-5, atol=1e-6)
