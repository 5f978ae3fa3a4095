"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every output element; they span several 16-token tiles,
several chunks and a ragged last chunk, every supported state size, both head
dims, fp32 and bf16 storage, groups, initial states, packed sequences (with
empty ones and starts in the middle of chunks), dt bias, the input-scaling
flag, and softplus on/off.  Every case is also run with D = None so that the
state-space part is not hidden under the D x skip term.  The full-size
workloads compare every (sequence, head) stream, in the same launch
configuration the benchmark times, and record the observed error.
"""
import numpy as np
import pytest

import ssd_synth
from checkers import dt_effective, rel_err
from parity import TOL, compare, fwd_into, record, run_gpu, run_oracle, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(name, **kw):
    extra = {k: kw.pop(k) for k in ("scales_input", "softplus", "dt_min", "dt_max", "dt_bias")
             if k in kw}
    inp = ssd_synth.random_case(**kw)
    for k, v in extra.items():
        if k == "dt_bias":
            v = np.full(inp.x.shape[2], v, np.float32)
        setattr(inp, k, v)
    inp.meta["case"] = name
    return inp


SMALL = [
    dict(name="f32_ragged_N32", seed=101, batch=2, seqlen=300, H=3, P=64, N=32, G=1, chunk=64,
         dtype="f32", with_init=True),
    dict(name="f32_N128_P128", seed=102, batch=1, seqlen=260, H=2, P=128, N=128, G=1, chunk=128,
         dtype="f32"),
    dict(name="f32_N256_Q256", seed=103, batch=1, seqlen=300, H=2, P=64, N=256, G=2, chunk=256,
         dtype="f32", with_init=True),
    dict(name="bf16_N128_Q256_G2", seed=104, batch=2, seqlen=700, H=4, P=64, N=128, G=2,
         chunk=256, dtype="bf16", with_init=True),
    dict(name="bf16_N16_P128", seed=105, batch=1, seqlen=333, H=2, P=128, N=16, G=1, chunk=128,
         dtype="bf16"),
    dict(name="bf16_N256", seed=106, batch=1, seqlen=520, H=2, P=64, N=256, G=1, chunk=256,
         dtype="bf16", with_init=True),
    dict(name="bf16_N64_P128_Q64", seed=107, batch=3, seqlen=130, H=2, P=128, N=64, G=2, chunk=64,
         dtype="bf16"),
    dict(name="bf16_N32_Q128", seed=108, batch=2, seqlen=129, H=4, P=64, N=32, G=4, chunk=128,
         dtype="bf16", with_init=True),
    dict(name="varlen_bf16_init", seed=109, batch=1, seqlen=1078, H=4, P=64, N=64, G=2, chunk=128,
         dtype="bf16", lengths=[0, 100, 1, 300, 0, 77, 600], with_init=True),
    dict(name="varlen_bf16_Q256", seed=110, batch=1, seqlen=1014, H=2, P=64, N=128, G=1,
         chunk=256, dtype="bf16", lengths=[5, 250, 256, 3, 500]),
    dict(name="varlen_f32_init", seed=111, batch=1, seqlen=329, H=2, P=64, N=32, G=1, chunk=64,
         dtype="f32", lengths=[64, 64, 1, 200], with_init=True),
    dict(name="varlen_bf16_N256_P128", seed=112, batch=1, seqlen=700, H=2, P=128, N=256, G=2,
         chunk=256, dtype="bf16", lengths=[300, 0, 17, 383], with_init=True),
    # packed sequences for the fused schedule: many short sequences (and empty
    # ones) inside single chunks, starts exactly at chunk starts, the input
    # scaling flag with a bias, several groups
    dict(name="varlen_bf16_tiny_seqs", seed=115, batch=1, seqlen=218, H=2, P=64, N=32, G=1,
         chunk=64, dtype="bf16", lengths=[8, 10, 0, 10, 6, 6, 8, 3, 12, 0, 3, 4, 7, 5, 1, 0, 0, 0, 1, 12, 2, 8, 9, 3, 3, 5, 3, 12, 2, 11, 10, 10, 1, 5, 8, 6, 8, 8, 8, 0], with_init=True),
    dict(name="varlen_bf16_chunk_aligned", seed=116, batch=1, seqlen=896, H=3, P=64, N=128, G=3,
         chunk=128, dtype="bf16", lengths=[128, 256, 0, 128, 1, 127, 256], with_init=True),
    dict(name="varlen_bf16_scaled_Q256", seed=117, batch=1, seqlen=777, H=2, P=64, N=16, G=2,
         chunk=256, dtype="bf16", lengths=[3, 400, 17, 0, 357], with_init=True,
         scales_input=True, dt_bias=0.3),
    dict(name="bf16_scaled_input_bias_nosoftplus", seed=113, batch=1, seqlen=400, H=2, P=64, N=64,
         G=1, chunk=128, dtype="bf16", scales_input=True, softplus=False, dt_bias=4.7,
         dt_min=0.0, dt_max=0.2),
    dict(name="f32_scaled_input_bias", seed=114, batch=2, seqlen=200, H=2, P=64, N=16, G=1,
         chunk=64, dtype="f32", scales_input=True, dt_bias=0.5, with_init=True),
]


def fused_supported(inp):
    """Shapes the fused single-pass schedule takes (the library refuses the others)."""
    return inp.dtype == "bf16" and inp.x.shape[3] == 64 and inp.B.shape[3] <= 128


def stream_supported(inp):
    """Shapes the stream-resident schedule takes: bf16, P = 64, dense rows, one
    group count for B and C."""
    return (inp.dtype == "bf16" and inp.x.shape[3] == 64 and inp.cu_seqlens is None
            and inp.B.shape[2] == inp.C.shape[2])


@pytest.mark.parametrize("spec", SMALL, ids=[c["name"] for c in SMALL])
@pytest.mark.parametrize("with_D", [True, False], ids=["D", "noD"])
@pytest.mark.parametrize("algo", ["chunked", "fused", "stream"])
def test_small_cases_elementwise(spec, with_D, algo):
    inp = _case(**dict(spec))
    if not with_D:
        inp.D = None
    if algo == "fused" and not fused_supported(inp):
        pytest.skip("shape outside the fused schedule (runs the chunked one)")
    if algo == "stream" and not stream_supported(inp):
        pytest.skip("shape outside the stream-resident schedule")
    say(f"case {spec['name']} D={with_D} algo={algo}")
    y, fin = run_gpu(inp, algo=algo)
    yr, fr = run_oracle(inp)
    ey, ef = compare(inp, y, fin, yr, fr)
    tol = TOL[inp.dtype]
    assert ey < tol, f"y error {ey:.3e} >= {tol}"
    assert ef < tol, f"final-state error {ef:.3e} >= {tol}"


def test_tiny_f32_workload():
    """The tiny fp32 workload: b1 L256 H2 P64 N16 G1 Q64, zero initial state."""
    inp = ssd_synth.make("tiny_f32")
    for with_D in (True, False):
        if not with_D:
            inp.D = None
        say(f"tiny_f32 D={with_D}")
        y, fin = run_gpu(inp)
        yr, fr = run_oracle(inp)
        ey, ef = compare(inp, y, fin, yr, fr)
        assert ey < 1e-4 and ef < 1e-4, (ey, ef)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_size_invariance(dtype):
    """Any chunk length gives the recurrence's result (section 6; appendix B.3.2)."""
    inp = _case("chunk_invariance", seed=120, batch=2, seqlen=777, H=2, P=64, N=64, G=1, chunk=64,
                dtype=dtype, with_init=True)
    yr, fr = run_oracle(inp)
    dev = to_device(inp)
    outs = []
    for Q in (64, 128, 256):
        say(f"chunk invariance {dtype} Q={Q}")
        y, fin = run_gpu(inp, chunk=Q, dev=dev)
        ey, ef = compare(inp, y, fin, yr, fr)
        assert ey < TOL[dtype] and ef < TOL[dtype], (Q, ey, ef)
        outs.append(y)
    # and the chunkings agree with each other more tightly than with the oracle
    assert rel_err(outs[0], outs[2]) < TOL[dtype]


def test_dt_cumsum_step():
    """dt preprocessing and per-chunk prefix sums of dt' A against numpy fp64."""
    import ssd_scan_amd as ssd

    inp = _case("dt_cumsum", seed=130, batch=2, seqlen=333, H=5, P=64, N=16, G=1, chunk=128,
                dtype="bf16")
    bias = np.linspace(-1, 1, 5).astype(np.float32)
    dev = to_device(inp)
    for softplus, lo, hi in ((True, 1e-3, 0.1), (False, 0.0, 1e30), (True, 0.0, 1e30)):
        say(f"dt_cumsum softplus={softplus} clamp=[{lo},{hi}]")
        dto, cso = ssd.dt_cumsum(dev["dt"], dev["A"], torch.from_numpy(bias).cuda(),
                                 chunk_size=128, softplus=softplus, dt_min=lo, dt_max=hi)
        torch.cuda.synchronize()
        dto, cso = dto.cpu().numpy(), cso.cpu().numpy()
        d = dt_effective(inp.dt, bias, softplus, lo, hi)  # (b, L, H)
        b, L, H = d.shape
        nc = (L + 127) // 128
        pad = np.zeros((b, nc * 128, H))
        pad[:, :L] = d
        dref = pad.reshape(b, nc, 128, H).transpose(0, 3, 1, 2)
        csref = np.cumsum(dref * inp.A.astype(np.float64)[None, :, None, None], axis=-1)
        np.testing.assert_allclose(dto, dref, rtol=2e-6, atol=1e-30)
        np.testing.assert_allclose(cso, csref, rtol=1e-5, atol=1e-5 * (1 + np.abs(csref).max()))


@pytest.mark.parametrize("algo", ["chunked", "fused", "stream"])
def test_deterministic_run_to_run(algo):
    inp = _case("determinism", seed=140, batch=2, seqlen=1000, H=4, P=64, N=128, G=1, chunk=256,
                dtype="bf16", with_init=True)
    dev = to_device(inp)
    say(f"determinism {algo}")
    y1, f1 = run_gpu(inp, dev=dev, algo=algo)
    y2, f2 = run_gpu(inp, dev=dev, algo=algo)
    assert np.array_equal(y1, y2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("N", [16, 32, 64, 128])
def test_fused_matches_oracle_every_instance(N, Q):
    """Every (N, Q) instance of the fused schedule, several chunks and a ragged tail,
    three B/C groups of two heads, with initial and final states."""
    inp = _case(f"fused_N{N}_Q{Q}", seed=150 + N + Q, batch=2, seqlen=3 * Q + 37, H=6, P=64, N=N,
                G=3, chunk=Q, dtype="bf16", with_init=True)
    for with_D in (True, False):
        if not with_D:
            inp.D = None
        say(f"fused N={N} Q={Q} D={with_D}")
        y, fin = run_gpu(inp, algo="fused")
        yr, fr = run_oracle(inp)
        ey, ef = compare(inp, y, fin, yr, fr)
        assert ey < 2e-2 and ef < 2e-2, (N, Q, with_D, ey, ef)


@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("N", [16, 32, 64, 128])
def test_fused_packed_every_instance(N, Q):
    """Every (N, Q) instance of the fused schedule on packed sequences: empty
    sequences, one ending mid-chunk, one starting exactly at a chunk start, a
    one-token sequence, one spanning chunks; initial and final states."""
    a = Q // 2 + 3
    lengths = [0, a, Q - a, 1, 0, Q + 20, 5]
    lengths.append(3 * Q + 37 - sum(lengths))
    inp = _case(f"fused_packed_N{N}_Q{Q}", seed=170 + N + Q, batch=1, seqlen=3 * Q + 37, H=4,
                P=64, N=N, G=2, chunk=Q, dtype="bf16", lengths=lengths, with_init=True)
    for with_D in (True, False):
        if not with_D:
            inp.D = None
        say(f"fused packed N={N} Q={Q} D={with_D}")
        y, fin = run_gpu(inp, algo="fused")
        yr, fr = run_oracle(inp)
        ey, ef = compare(inp, y, fin, yr, fr)
        assert ey < 2e-2 and ef < 2e-2, (N, Q, with_D, ey, ef)


@pytest.mark.parametrize("Q", [64, 128, 256])
@pytest.mark.parametrize("N,P", [(16, 64), (32, 64), (64, 64), (128, 64), (256, 64), (16, 128),
                                 (32, 128), (64, 128), (128, 128), (256, 128)])
def test_chunked_bf16_every_instance(N, P, Q):
    """Every bf16 (N, P, Q) instance of the chunked schedule (streaming chunk
    state and chunk scan where N P <= 16384, register-staged kernels for N = 256
    at P = 128) on packed sequences with empty sequences, a chunk-aligned start,
    a one-token sequence, initial and final states."""
    lengths = [0, Q, 5, 1, 0, 2 * Q - 3]
    lengths.append(3 * Q + 29 - sum(lengths))
    inp = _case(f"chunked_N{N}_P{P}_Q{Q}", seed=400 + N + P + Q, batch=1, seqlen=3 * Q + 29, H=2,
                P=P, N=N, G=2, chunk=Q, dtype="bf16", lengths=lengths, with_init=True)
    for with_D in (True, False):
        if not with_D:
            inp.D = None
        say(f"chunked N={N} P={P} Q={Q} D={with_D}")
        y, fin = run_gpu(inp, algo="chunked")
        yr, fr = run_oracle(inp)
        ey, ef = compare(inp, y, fin, yr, fr)
        assert ey < 2e-2 and ef < 2e-2, (N, P, Q, with_D, ey, ef)


@pytest.mark.parametrize("mode", [0, 1, 2], ids=["flags_early", "flags_late", "tagged"])
@pytest.mark.parametrize("N,Q", [(32, 64), (128, 256)])
def test_fused_every_handoff_placement(N, Q, mode, monkeypatch):
    """The three hand-off placements of the fused schedule (flag before the
    chunk states, flag after them, tagged ring), forced through
    SSD_FUSED_HANDOFF, on batch rows with initial and final states and on
    packed sequences with chunk-aligned starts and empty sequences."""
    monkeypatch.setenv("SSD_FUSED_HANDOFF", str(mode))
    rows = _case(f"handoff_rows_N{N}_Q{Q}", seed=180 + N + Q, batch=3, seqlen=4 * Q + 19, H=3,
                 P=64, N=N, G=1, chunk=Q, dtype="bf16", with_init=True)
    lengths = [Q, 0, Q, 7, 2 * Q - 7, 0, Q + 11]
    packed = _case(f"handoff_packed_N{N}_Q{Q}", seed=190 + N + Q, batch=1, seqlen=sum(lengths),
                   H=3, P=64, N=N, G=3, chunk=Q, dtype="bf16", lengths=lengths, with_init=True)
    for inp in (rows, packed):
        say(f"hand-off placement {mode}: {inp.meta['case']}")
        y, fin = run_gpu(inp, algo="fused")
        yr, fr = run_oracle(inp)
        ey, ef = compare(inp, y, fin, yr, fr)
        assert ey < 2e-2 and ef < 2e-2, (inp.meta["case"], mode, ey, ef)


PATTERNS = [("multi_contract", 1, 8), ("multi_expand", 8, 1), ("mixed", 2, 4)]


@pytest.mark.parametrize("pattern,G,Gc", PATTERNS, ids=[p[0] for p in PATTERNS])
@pytest.mark.parametrize("algo,dtype,N,P", [("fused", "bf16", 64, 64), ("chunked", "bf16", 128, 64),
                                            ("chunked", "bf16", 256, 64), ("chunked", "f32", 32, 128)],
                         ids=["fused", "chunked_bf16", "chunked_bf16_N256", "chunked_f32"])
@pytest.mark.parametrize("packed", [False, True], ids=["rows", "packed"])
def test_head_patterns(pattern, G, Gc, algo, dtype, N, P, packed):
    """Section 7.2 head patterns: B and C heads shared by different numbers of
    x heads (C with its own group count), in every schedule."""
    if packed:
        inp = _case(f"{pattern}_packed", seed=210 + G + 3 * Gc, batch=1, seqlen=700, H=8, P=P, N=N,
                    G=G, Gc=Gc, chunk=128, dtype=dtype, lengths=[128, 0, 301, 271],
                    with_init=True)
    else:
        inp = _case(f"{pattern}_rows", seed=220 + G + 3 * Gc, batch=2, seqlen=500, H=8, P=P, N=N,
                    G=G, Gc=Gc, chunk=128, dtype=dtype, with_init=True)
    say(f"head pattern {pattern} {algo} {dtype} N={N} packed={packed}")
    y, fin = run_gpu(inp, algo=algo)
    yr, fr = run_oracle(inp)
    ey, ef = compare(inp, y, fin, yr, fr)
    tol = TOL[dtype]
    assert ey < tol and ef < tol, (ey, ef)


def test_handoff_give_up_is_reported(monkeypatch):
    """A hand-off wait that gives up is reported under SSD_VALIDATE=1 and
    leaves NaN in the outputs that depend on the missing state.  The host
    lowers the waits' bound to zero sleeps (every kernel still ends): on one
    long stream a chunk reaches its wait before its predecessor has published,
    so the call must return SSD_ERR_HIP; with the default bound the same call
    succeeds and matches the oracle."""
    import ssd_scan_amd as ssd

    inp = _case("give_up", seed=191, batch=1, seqlen=64 * 40, H=1, P=64, N=32, G=1, chunk=64,
                dtype="bf16")
    monkeypatch.setenv("SSD_VALIDATE", "1")
    say("hand-off give-up reported")
    for mode in ("0", "1", "2"):
        monkeypatch.setenv("SSD_FUSED_HANDOFF", mode)
        monkeypatch.setenv("SSD_SPIN_LIMIT", "0")
        y, err = fwd_into(inp, "fused")
        assert err is not None and err.status == ssd.SSD_ERR_HIP, mode
        # the chunks whose wait gave up computed from a NaN state: their
        # outputs (and everything downstream of them) are NaN, not silently wrong
        assert np.isnan(y).any(), mode
        monkeypatch.delenv("SSD_SPIN_LIMIT")
        y, fin = run_gpu(inp, algo="fused")
        yr, fr = run_oracle(inp)
        ey, ef = compare(inp, y, fin, yr, fr)
        assert ey < 2e-2 and ef < 2e-2, (mode, ey, ef)


GUARD_CASES = [
    dict(name="guard_packed_bf16", seed=150, batch=1, seqlen=333, H=2, P=64, N=32, G=1, chunk=128,
         dtype="bf16", lengths=[100, 0, 233], with_init=True),
    dict(name="guard_rows_bf16_N256", seed=151, batch=2, seqlen=300, H=2, P=64, N=256, G=1,
         chunk=256, dtype="bf16", with_init=True),
    dict(name="guard_rows_f32_P128", seed=152, batch=2, seqlen=131, H=3, P=128, N=64, G=1,
         chunk=64, dtype="f32", with_init=True),
    dict(name="guard_packed_f32", seed=153, batch=1, seqlen=200, H=2, P=64, N=16, G=2, chunk=64,
         dtype="f32", lengths=[64, 1, 0, 135], with_init=True),
]


@pytest.mark.parametrize("algo", ["auto", "fused", "chunked"])
@pytest.mark.parametrize("spec", GUARD_CASES, ids=[c["name"] for c in GUARD_CASES])
def test_outputs_stay_in_bounds(spec, algo):
    """Canaries around y and the final states are left untouched (packed and
    dense inputs, ragged last chunks, every schedule that takes the shape)."""
    import ssd_scan_amd as ssd

    inp = _case(**dict(spec))
    if algo == "fused" and not fused_supported(inp):
        pytest.skip("shape outside the fused schedule")
    dev = to_device(inp)
    pad = 4096
    ydt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    ybuf = torch.full((inp.x.size + 2 * pad,), -7.0, dtype=ydt, device="cuda")
    fbuf = torch.full((inp.initial_states.size + 2 * pad,), -7.0, dtype=torch.float32,
                      device="cuda")
    y = ybuf[pad:pad + inp.x.size].view(inp.x.shape)
    fin = fbuf[pad:pad + inp.initial_states.size].view(inp.initial_states.shape)
    say(f"guard bands {spec['name']} {algo}")
    ssd.fwd(**dev, chunk_size=inp.chunk, dt_min=inp.dt_min, dt_max=inp.dt_max, out=y,
            final_states=fin, algo=algo)
    torch.cuda.synchronize()
    for buf in (ybuf, fbuf):
        assert torch.all(buf[:pad] == -7.0) and torch.all(buf[-pad:] == -7.0)
    yr, fr = run_oracle(inp)
    ey, ef = compare(inp, y.float().cpu().numpy(), fin.cpu().numpy(), yr, fr)
    assert ey < TOL[inp.dtype] and ef < TOL[inp.dtype], (ey, ef)


def test_empty_sequences_only_and_zero_length():
    import ssd_scan_amd as ssd

    # no tokens at all: final states equal the initial states
    init = torch.randn(3, 2, 16, 64, device="cuda")
    x = torch.zeros(3, 0, 2, 64, device="cuda")
    y, fin = ssd.fwd(x, torch.zeros(3, 0, 2, device="cuda"), -torch.ones(2, device="cuda"),
                     torch.zeros(3, 0, 1, 16, device="cuda"), torch.zeros(3, 0, 1, 16,
                                                                              device="cuda"),
                     initial_states=init, chunk_size=64, return_final_states=True)
    torch.cuda.synchronize()
    assert torch.equal(fin, init)


# ---------------------------------------------------------------- full-size workloads
_LAST_ORACLE = {}


def _full(name, with_D=True, algo="auto"):
    """Every (sequence, head) stream of a full-size workload against the oracle
    (the oracle runs all of them, OpenMP over the host cores), in the launch
    configuration the benchmark times; the observed errors are recorded.  The
    oracle's result for the last workload is kept for the next schedule."""
    inp = ssd_synth.make(name)
    if not with_D:
        inp.D = None
    say(f"workload {name} D={with_D} algo={algo} (every stream)")
    y, fin = run_gpu(inp, want_final=inp.want_final, algo=algo)
    key = (name, with_D)
    if key not in _LAST_ORACLE:
        _LAST_ORACLE.clear()
        _LAST_ORACLE[key] = run_oracle(inp, want_final=inp.want_final)
    yr, fr = _LAST_ORACLE[key]
    ey, ef = compare(inp, y, fin, yr, fr)
    record(f"{name} D={with_D} algo={algo}", y=ey, final=ef)
    assert np.isfinite(y).all()
    tol = TOL[inp.dtype]
    assert ey < tol, f"{name}: y error {ey:.3e}"
    if inp.want_final:
        assert ef < tol, f"{name}: final-state error {ef:.3e}"
    return ey, ef


@pytest.mark.parametrize("algo", ["auto", "stream", "fused", "chunked"])
@pytest.mark.parametrize("with_D", [True, False], ids=["D", "noD"])
@pytest.mark.parametrize("name", ["mamba2_130m", "mamba2_2p7b"])
def test_full_size_dense_workloads(name, with_D, algo):
    _full(name, with_D, algo)


def test_full_size_deterministic_run_to_run():
    """Two launches of the 2.7B-shaped layer in the benchmark's configuration
    give the same bits (range hand-offs and tickets do not change the
    arithmetic)."""
    inp = ssd_synth.make("mamba2_2p7b")
    dev = to_device(inp)
    say("full-size determinism mamba2_2p7b")
    y1, _ = run_gpu(inp, dev=dev, want_final=False)
    y2, _ = run_gpu(inp, dev=dev, want_final=False)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("algo", ["auto", "stream"])
@pytest.mark.parametrize("L", ssd_synth.SWEEP_L)
@pytest.mark.parametrize("N", ssd_synth.SWEEP_N)
def test_full_size_sweep(L, N, algo):
    _full(f"sweep_L{L}_N{N}", algo=algo)


@pytest.mark.parametrize("with_D", [True, False], ids=["D", "noD"])
def test_full_size_varlen(with_D):
    _full("varlen_80h", with_D)
