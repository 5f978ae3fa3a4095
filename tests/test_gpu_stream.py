"""GPU parity of the stream-resident schedule (``algo="stream"``) against the
fp64 oracle, through the C ABI.

The schedule walks runs of chunks of a (row, head) with the state in
registers, composes the state entering each run from the run in front of it,
shares the masked C B^T of a chunk between the heads of a B/C group and feeds
the matrix cores fp16 operands scaled per block by powers of two.  The cases
below cover every (N, Q) instance with several chunks and a ragged tail, every
forced number of runs per stream (one run, two, uneven, one chunk per run),
initial and final states, D and no D, dt bias with and without softplus, the
input-scaling flag, decays strong enough that a 16-token block spans more than
88 nats, inputs far outside fp16 range in both directions, and B = 0 (y must
be D x exactly).
"""
import numpy as np
import pytest

import ssd_synth
from parity import TOL, compare, fwd_into, record, run_gpu, run_oracle, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(name, seed, batch, seqlen, H, N, G, chunk, with_init=True, **extra):
    inp = ssd_synth.random_case(seed, batch, seqlen, H, 64, N, G, chunk=chunk, dtype="bf16",
                                with_init=with_init)
    for k, v in extra.items():
        if k == "dt_bias":
            v = np.full(H, v, np.float32)
        setattr(inp, k, v)
    inp.meta["case"] = name
    return inp


def _check(inp, label, tol=2e-2):
    y, fin = run_gpu(inp, algo="stream")
    yr, fr = run_oracle(inp)
    ey, ef = compare(inp, y, fin, yr, fr)
    record(label, y=ey, final=ef)
    assert np.isfinite(y).all(), label
    assert ey < tol, f"{label}: y error {ey:.3e}"
    assert ef < tol, f"{label}: final-state error {ef:.3e}"


@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
def test_stream_every_instance(N, Q):
    """Every (N, Q) instance: several chunks and a ragged tail, three B/C groups
    of two heads, initial and final states, with and without D."""
    inp = _case(f"stream_N{N}_Q{Q}", 600 + N + Q, 2, 3 * Q + 37, 6, N, 3, Q)
    for with_D in (True, False):
        if not with_D:
            inp.D = None
        say(f"stream N={N} Q={Q} D={with_D}")
        _check(inp, f"stream N={N} Q={Q} D={with_D}")


@pytest.mark.parametrize("segments", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("N,Q", [(32, 64), (128, 256), (256, 128)])
def test_stream_runs_per_stream(N, Q, segments, monkeypatch):
    """The runs of chunks a stream is cut into, forced through
    SSD_STREAM_SEGMENTS: one run, two, uneven runs, and one chunk per run (every
    run composes the state entering it from the run in front)."""
    monkeypatch.setenv("SSD_STREAM_SEGMENTS", str(segments))
    inp = _case(f"runs_N{N}_Q{Q}_S{segments}", 650 + N + Q + segments, 2, 9 * Q + 5, 3, N, 1, Q)
    for with_init in (True, False):
        if not with_init:
            inp.initial_states = None
        say(f"stream runs={segments} N={N} Q={Q} init={with_init}")
        _check(inp, f"stream runs={segments} N={N} Q={Q} init={with_init}")


@pytest.mark.parametrize("units", [9, 10, 17, 29, 1000])
@pytest.mark.parametrize("N,Q", [(64, 64), (128, 256)])
def test_stream_range_mode(N, Q, units, monkeypatch):
    """Range mode, forced through SSD_STREAM_RANGE: each workgroup walks a run
    of `units` (stream, chunk) units of the stream-major order (a stream's
    tail, whole streams, the head of the next one); a tail starts from the
    state published by the workgroup that walked the head.  Seven streams of
    nine chunks (the last one ragged): ranges of exactly one stream, one
    chunk more, uneven heads and tails, and everything in one workgroup."""
    monkeypatch.setenv("SSD_STREAM_RANGE", str(units))
    inp = _case(f"range_N{N}_Q{Q}_R{units}", 760 + N + Q + units, 1, 9 * Q - 11, 7, N, 1, Q)
    for with_init in (True, False):
        if not with_init:
            inp.initial_states = None
        say(f"stream range={units} N={N} Q={Q} init={with_init}")
        _check(inp, f"stream range={units} N={N} Q={Q} init={with_init}")


def test_stream_range_mode_matches_one_walk(monkeypatch):
    """A range split changes nothing in the arithmetic: every chunk is walked
    once, in order, from the same state, so the outputs are bit-identical to
    one workgroup per stream."""
    inp = _case("range_bits", 790, 2, 5 * 256 - 3, 5, 128, 1, 256)
    dev = to_device(inp)
    monkeypatch.setenv("SSD_STREAM_SEGMENTS", "1")
    y1, f1 = run_gpu(inp, dev=dev, algo="stream")
    monkeypatch.delenv("SSD_STREAM_SEGMENTS")
    for units in (5, 7, 12):
        monkeypatch.setenv("SSD_STREAM_RANGE", str(units))
        say(f"stream range bits units={units}")
        y2, f2 = run_gpu(inp, dev=dev, algo="stream")
        assert np.array_equal(y1, y2) and np.array_equal(f1, f2), units


@pytest.mark.parametrize("variant", ["bias_softplus", "bias_nosoftplus", "scaled", "scaled_bias"])
def test_stream_dt_options(variant):
    kw = {
        "bias_softplus": dict(dt_bias=0.7),
        "bias_nosoftplus": dict(dt_bias=4.7, softplus=False, dt_min=0.0, dt_max=0.2),
        "scaled": dict(scales_input=True),
        "scaled_bias": dict(scales_input=True, dt_bias=-0.4),
    }[variant]
    inp = _case(f"dt_{variant}", 680, 2, 600, 4, 64, 2, 256, **kw)
    say(f"stream dt options {variant}")
    _check(inp, f"stream dt {variant}")


def test_stream_strong_decay():
    """dt up to 6 with |A| up to 16: a 16-token block can span hundreds of nats,
    every per-token decay underflows or nearly so."""
    inp = _case("strong_decay", 690, 1, 700, 4, 64, 1, 256, dt_max=6.0)
    inp.dt = ssd_synth.round_to_bf16(inp.dt + 6.0)
    say("stream strong decay")
    _check(inp, "stream strong decay")


@pytest.mark.parametrize("scale", [1e-12, 1e12])
def test_stream_out_of_fp16_range(scale):
    """x and C scaled far outside fp16 range (1e12 and 1e-12), B the other way:
    the block scales keep every matrix-core operand in range."""
    inp = _case(f"range_{scale:g}", 700, 2, 520, 2, 128, 1, 256)
    inp.x = ssd_synth.round_to_bf16(inp.x * scale)
    inp.C = ssd_synth.round_to_bf16(inp.C * scale)
    inp.B = ssd_synth.round_to_bf16(inp.B / scale)
    say(f"stream operand range x{scale:g}")
    _check(inp, f"stream range {scale:g}")


def test_stream_zero_B_gives_D_x_exactly():
    """B = 0 and a zero initial state: the state stays zero and y = D x, each
    element rounded once to bf16."""
    inp = _case("zero_B", 710, 2, 300, 3, 64, 1, 128, with_init=False)
    inp.B = np.zeros_like(inp.B)
    y, fin = run_gpu(inp, algo="stream")
    ref = inp.x.astype(np.float32) * inp.D[None, None, :, None]
    expect = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(y, expect.astype(np.float64))
    assert not np.any(fin)


def test_stream_and_fused_both_within_tolerance():
    """The stream schedule and the fused schedule agree within the bf16 bound on
    the same inputs (both against the oracle, and with each other)."""
    inp = _case("vs_fused", 720, 2, 1000, 4, 128, 1, 256)
    yr, fr = run_oracle(inp)
    dev = to_device(inp)
    ys, fs = run_gpu(inp, algo="stream", dev=dev)
    yf, ff = run_gpu(inp, algo="fused", dev=dev)
    for y, fin in ((ys, fs), (yf, ff)):
        ey, ef = compare(inp, y, fin, yr, fr)
        assert ey < TOL["bf16"] and ef < TOL["bf16"], (ey, ef)


def test_stream_deterministic_run_to_run():
    inp = _case("determinism", 730, 2, 1000, 4, 128, 1, 256)
    dev = to_device(inp)
    say("stream determinism")
    y1, f1 = run_gpu(inp, dev=dev, algo="stream")
    y2, f2 = run_gpu(inp, dev=dev, algo="stream")
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)


def test_stream_outputs_stay_in_bounds(monkeypatch):
    """Canaries around y and the final states are left untouched (ragged last
    chunk, several runs per stream)."""
    import ssd_scan_amd as ssd

    monkeypatch.setenv("SSD_STREAM_SEGMENTS", "3")
    inp = _case("guard", 740, 2, 333, 2, 32, 1, 64)
    dev = to_device(inp)
    pad = 4096
    ybuf = torch.full((inp.x.size + 2 * pad,), -7.0, dtype=torch.bfloat16, device="cuda")
    fbuf = torch.full((inp.initial_states.size + 2 * pad,), -7.0, dtype=torch.float32,
                      device="cuda")
    y = ybuf[pad:pad + inp.x.size].view(inp.x.shape)
    fin = fbuf[pad:pad + inp.initial_states.size].view(inp.initial_states.shape)
    say("stream guard bands")
    ssd.fwd(**dev, chunk_size=64, dt_min=inp.dt_min, dt_max=inp.dt_max, out=y, final_states=fin,
            algo="stream")
    torch.cuda.synchronize()
    for buf in (ybuf, fbuf):
        assert torch.all(buf[:pad] == -7.0) and torch.all(buf[-pad:] == -7.0)
    yr, fr = run_oracle(inp)
    ey, ef = compare(inp, y.float().cpu().numpy(), fin.cpu().numpy(), yr, fr)
    assert ey < 2e-2 and ef < 2e-2


def test_stream_give_up_poisons_outputs(monkeypatch):
    """A segment-entry wait that gives up is reported under SSD_VALIDATE=1 and
    leaves non-finite values in the outputs that depend on the missing state.  The host
    lowers the waits' bound to zero sleeps (every kernel still ends) and cuts
    one stream into 64 one-chunk segments: the entering state of a segment is
    published only after the segment in front has received its own, so the
    later segments reach their waits first and give up.  With the default
    bound the same call matches the oracle."""
    import ssd_scan_amd as ssd

    inp = _case("give_up", 795, 1, 64 * 64, 1, 32, 1, 64)
    monkeypatch.setenv("SSD_STREAM_SEGMENTS", "64")
    monkeypatch.setenv("SSD_VALIDATE", "1")
    monkeypatch.setenv("SSD_SPIN_LIMIT", "0")
    say("stream give-up reported")
    y, err = fwd_into(inp, "stream")
    assert err is not None and err.status == ssd.SSD_ERR_HIP
    assert not np.isfinite(y).all()
    monkeypatch.delenv("SSD_SPIN_LIMIT")
    _check(inp, "stream give-up case, default bound")
