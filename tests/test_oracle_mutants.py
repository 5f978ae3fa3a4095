"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a plausible slip in ``oracle/ssd_ref.c`` (a dropped term, a wrong
sign, a wrong index, a transposed operand, a skipped preprocessing step).  The
mutant source is compiled on the CPU into a temporary library and the pins of
``test_oracle_pins.py`` are run against it; a mutant that passes every pin
would show a hole in the pins.
"""
import os
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

MUTANTS = {
    "no_decay": ("Sn[p] = a * Sn[p] + bn * (double)xt[p];", "Sn[p] = Sn[p] + bn * (double)xt[p];"),
    "decay_sign": ("const double a = exp(dtv * Ah);", "const double a = exp(-dtv * Ah);"),
    "no_skip": ("yt[p] = Dh * (double)xt[p];", "yt[p] = 0.0;"),
    "group_modulo": ("const int64_t g = h / (H / G), gc = h / (H / Gc);",
                     "const int64_t g = h % G, gc = h % Gc;"),
    "c_uses_b_group": ("const float* Ct = C + (t * Gc + gc) * N;",
                       "const float* Ct = C + (t * Gc + g % Gc) * N;"),
    "swap_B_C": ("const float* Bt = B + (t * G + g) * N;\n    const float* Ct = C + (t * Gc + gc) * N;",
                 "const float* Bt = C + (t * Gc + gc) * N;\n    const float* Ct = B + (t * G + g) * N;"),
    "init_ignored": ("S[i] = (double)init[i];", "S[i] = 0.0;"),
    "softplus_sign": ("log1p(exp(-fabs(v)))", "log1p(exp(fabs(v)))"),
    "softplus_no_max": ("fmax(v, 0.0) + log1p", "log1p"),
    "no_clamp": ("dtv = fmin(fmax(dtv, dt_min), dt_max);", ""),
    "no_bias": ("double dtv = (double)dt[t * H + h] + bias;", "double dtv = (double)dt[t * H + h];"),
    "scaling_ignored": ("? dtv : 1.0;", "? 1.0 : 1.0;"),
    "state_transposed_readout": ("yt[p] += cn * Sn[p];", "yt[p] += cn * S[(p * N + n) % (N * P)];"),
    "x_head_is_group": ("const float* xt = x + (t * H + h) * P;", "const float* xt = x + (t * H + g) * P;"),
    "readout_before_update": (
        "    /* state update: S[n,p] = a * S[n,p] + in_scale * B[n] * x[p] */\n"
        "    for (int64_t n = 0; n < N; ++n) {\n"
        "      const double bn = in_scale * (double)Bt[n];\n"
        "      double* Sn = S + n * P;\n"
        "      for (int64_t p = 0; p < P; ++p) Sn[p] = a * Sn[p] + bn * (double)xt[p];\n"
        "    }\n", ""),
    "last_token_skipped": ("for (int64_t t = tok0; t < tok0 + len; ++t)",
                           "for (int64_t t = tok0; t + 1 < tok0 + len; ++t)"),
    "varlen_no_reset": ("const int64_t tok0 = cu_seqlens ? cu_seqlens[s] : s * seqlen;\n"
                        "      const int64_t len = cu_seqlens ? cu_seqlens[s + 1] - cu_seqlens[s] : seqlen;",
                        "const int64_t tok0 = cu_seqlens ? 0 : s * seqlen;\n"
                        "      const int64_t len = cu_seqlens ? cu_seqlens[s + 1] : seqlen;"),
}

# slips in the backward pass, caught by the backward pins
BWD_MUTANTS = {
    "bwd_no_adjoint_decay": ("for (int64_t i = 0; i < NP; ++i) g[i] *= a;", ""),
    "bwd_dl_uses_current_state": ("gS += g[i] * prev[i];", "gS += g[i] * cur[i];"),
    "bwd_dC_uses_previous_state": ("sd += cur[n * P + p] * (double)dyt[p];",
                                   "sd += prev[n * P + p] * (double)dyt[p];"),
    "bwd_no_sigmoid": ("gate *= ref_sigmoid(pre);", ""),
    "bwd_dB_unscaled": ("dBt[n] = sc * gx;", "dBt[n] = gx;"),
    "bwd_no_scaled_dt_term": ("if (flags & REF_FLAG_SCALES_INPUT) ddtp += gBx;", ""),
    "bwd_dA_without_dt": ("dA_acc += dl * dtv;", "dA_acc += dl;"),
    "bwd_group_sum_modulo": ("dB[(t * G + h / (H / G)) * N + n]", "dB[(t * G + h % G) * N + n]"),
    "bwd_clamp_gate_open": ("(act >= dt_min && act <= dt_max) ? 1.0 : 0.0", "1.0"),
}


def _bwd_battery():
    import test_oracle_bwd_pins as bp
    out = [(f"fd[{s['seed']}]", bp.test_bwd_matches_central_differences, dict(spec=s))
           for s in bp.FD_CASES]
    out += [(f"autograd[{s['seed']}]", bp.test_bwd_matches_autograd_of_quadratic_form, dict(spec=s))
            for s in bp.AUTOGRAD_CASES]
    return out


def _pin_battery():
    out = [("golden", pins.test_golden_worked_examples, {})]
    for i, case in enumerate(pins.QUAD_CASES):
        for si in (False, True):
            out.append((f"quadratic[{i},{si}]", pins.test_quadratic_form,
                        dict(case=case, scales_input=si)))
    for name in ("test_quadratic_form_strong_decay_and_growth",
                 "test_a_equals_one_is_causal_linear_attention",
                 "test_a_equals_zero_keeps_only_the_current_token",
                 "test_zero_input_is_cumulative_product_of_the_initial_state",
                 "test_zero_B_or_C_leaves_the_skip_term", "test_without_D_there_is_no_skip",
                 "test_linearity_in_x_and_initial_state", "test_varlen_equals_separate_runs",
                 "test_varlen_is_recurrence_with_zero_decay_at_starts",
                 "test_group_broadcast_equals_replicated_heads",
                 "test_input_scaling_flag_is_scaling_x_by_dt",
                 "test_dt_preprocessing_softplus_bias_and_clamp"):
        out.append((name, getattr(pins, name), {}))
    out.append(("chunked[16]", pins.test_block_decomposition_matches_recurrence, dict(Q=16)))
    for G, Gc in ((1, 6), (2, 3)):
        out.append((f"groups[{G},{Gc}]", pins.test_separate_B_and_C_groups_equal_replicated_heads,
                    dict(G=G, Gc=Gc)))
    return out


BWD_MARK = "/*\n * Backward pass (gradients)"


def _mutant_source(name):
    full = open(oracle.SOURCE).read()
    cut = full.index(BWD_MARK)
    # forward slips go into the forward code only, backward slips into the backward code
    if name in BWD_MUTANTS:
        head, src = full[:cut], full[cut:]
    else:
        src, head = full[:cut], full[cut:]
    old, new = {**MUTANTS, **BWD_MUTANTS}[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    src = src.replace(old, new)
    if name == "readout_before_update":
        # re-insert the removed state update after the readout
        upd = MUTANTS[name][0]
        anchor = "      for (int64_t p = 0; p < P; ++p) yt[p] += cn * Sn[p];\n    }\n"
        assert src.count(anchor) == 1
        src = src.replace(anchor, anchor + upd)
    return head + src if name in BWD_MUTANTS else src + head


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, f"mut_{name}.c")
        open(path, "w").write(_mutant_source(name))
        lib = oracle.load(oracle.compile_oracle(path, os.path.join(tmp, f"libmut_{name}.so")))
        caught = []
        for label, fn, kw in _pin_battery():
            try:
                fn(lib, **kw)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(label)
        assert caught, f"mutant {name} passed every pin"


def test_unmutated_source_passes_the_battery(oracle_lib):
    for label, fn, kw in _pin_battery():
        fn(oracle_lib, **kw)


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, f"mut_{name}.c")
        open(path, "w").write(_mutant_source(name))
        lib = oracle.load(oracle.compile_oracle(path, os.path.join(tmp, f"libmut_{name}.so")))
        caught = []
        for label, fn, kw in _bwd_battery():
            try:
                fn(lib, **kw)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(label)
        assert caught, f"mutant {name} passed every backward pin"


def test_unmutated_source_passes_the_backward_battery(oracle_lib):
    for label, fn, kw in _bwd_battery():
        fn(oracle_lib, **kw)
