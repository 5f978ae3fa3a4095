"""C ABI checks that need no GPU: exports, struct layout, host-side validation.

Every invalid call below must be rejected by host validation with its own
status before anything is enqueued; the pointers passed are fake and are never
dereferenced (a HIP call on this GPU-less host would return SSD_ERR_HIP).
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

import ssd_scan_amd as ssd

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "ssd.h")
FAKE = 0x7F0000001000  # never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)  # drop comments
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["ssd_bwd", "ssd_bwd_events", "ssd_bwd_workspace_size",
                                    "ssd_dt_cumsum", "ssd_fwd", "ssd_fwd_events",
                                    "ssd_fwd_noalloc", "ssd_status_string", "ssd_step",
                                    "ssd_version",
                                    "ssd_workspace_size"]


def test_library_exports_every_declared_symbol():
    lib = ssd.library()
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
        getattr(lib, name)  # resolvable through the loader too


def test_problem_struct_layout():
    # 8 x int64, then int32 dtype, uint32 flags, float dt_min, float dt_max, int32 algo, int32
    assert ctypes.sizeof(ssd.SsdProblem) == 88
    assert ssd.SsdProblem.dtype.offset == 64 and ssd.SsdProblem.ngroups_c.offset == 84


def test_version_and_status_strings():
    assert "gfx950" in ssd.version()
    names = {ssd.status_string(s) for s in range(5)}
    assert len(names) == 5
    assert ssd.status_string(99) == "unknown status"


def good(**kw):
    args = dict(batch=2, seqlen=512, nheads=4, headdim=64, dstate=64, ngroups=2, chunk_size=128)
    args.update(kw)
    extra = {k: args.pop(k) for k in list(args) if k not in
             ("batch", "seqlen", "nheads", "headdim", "dstate", "ngroups", "chunk_size")}
    return ssd.make_problem(**args, **extra)


def call(p, ws_bytes=None, cu=None, x=FAKE, y=FAKE, ws=FAKE, prob_ptr=True):
    lib = ssd.library()
    if ws_bytes is None:
        ws_bytes = ssd.workspace_size(p)
    return lib.ssd_fwd(ctypes.byref(p) if prob_ptr else None, x, FAKE, FAKE, FAKE, FAKE, None,
                       None, None, cu, y, None, ws, ws_bytes, None)


def test_auto_schedule_choice():
    """AUTO takes the stream-resident schedule in range mode (enough chunks
    for every resident workgroup to walk whole streams; that needs a device,
    so not here).  Otherwise, among dense bf16 rows at P = 64: the stream
    schedule for N >= 64 on very long (>= 256 chunks) or very short (<= 2
    chunks) streams, for N = 256 from 64 chunks on (chunked below), the fused
    pass elsewhere; shapes outside the stream schedule as before (fused,
    chunked for small problems with N >= 64).  The workspace size tells which
    schedule a problem resolves to."""
    def picks(**kw):
        auto = ssd.workspace_size(good(**kw))
        sizes = {ssd.workspace_size(good(algo="fused", **kw)): "fused",
                 ssd.workspace_size(good(algo="chunked", **kw)): "chunked"}
        stream = ssd.workspace_size(good(algo="stream", **kw))
        if stream:
            sizes[stream] = "stream"
        return sizes[auto]

    long = dict(batch=1, nheads=2, ngroups=1, seqlen=256 * 128)   # 256 chunks of 128
    short = dict(batch=1, nheads=2, ngroups=1, seqlen=2 * 128)    # 2 chunks
    mid = dict(batch=1, nheads=2, ngroups=1, seqlen=32 * 128)     # 32 chunks
    for n in (64, 128):
        assert picks(dstate=n, **long) == "stream"
        assert picks(dstate=n, **short) == "stream"
        assert picks(dstate=n, **mid) == "fused"
    for n in (16, 32):
        assert picks(dstate=n, **long) == "fused"
        assert picks(dstate=n, **short) == "fused"
    assert picks(dstate=256, **long) == "stream"
    assert picks(dstate=256, **mid) == "chunked"
    assert picks(dstate=256, batch=1, nheads=2, ngroups=1, seqlen=64 * 128) == "stream"
    # separate C groups: fused (or chunked for small problems with N >= 64)
    assert picks(dstate=32, ngroups_c=4) == "fused"
    assert picks(dstate=64, ngroups_c=4) == "chunked"
    assert picks(batch=8, nheads=16, ngroups=4, ngroups_c=16, dstate=128) == "fused"
    # P = 128 and fp32 storage: chunked
    assert picks(dstate=32, headdim=128) == "chunked"
    assert picks(dstate=32, bf16=False) == "chunked"


def test_workspace_size():
    p = good(algo="chunked")
    n = ssd.workspace_size(p)
    assert n > 0 and n % 256 == 0
    # chunk states of every chunk: grows with the sequence
    assert ssd.workspace_size(good(seqlen=1024, algo="chunked")) > n
    # the fused single pass keeps a two-slot hand-off ring per (row, head)
    # (two words per state value) and two floats per (token, head), no chunk
    # states: it grows more slowly with the sequence
    f = ssd.workspace_size(good(algo="fused"))
    f2 = ssd.workspace_size(good(seqlen=4096, algo="fused"))
    assert 0 < f < f2 < ssd.workspace_size(good(seqlen=4096, algo="chunked"))
    assert f2 - f < ssd.workspace_size(good(seqlen=4096, algo="chunked")) - n
    # shapes outside the fused schedule are rejected when it is requested
    assert ssd.workspace_size(good(algo="fused", bf16=False)) == 0
    assert call(good(algo="fused", dstate=256), ws_bytes=1 << 30) == ssd.SSD_ERR_UNSUPPORTED
    assert ssd.workspace_size(good(ngroups=3)) == 0  # invalid problem
    assert ssd.library().ssd_workspace_size(None) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ngroups=3), ssd.SSD_ERR_INVALID_ARG),
    (dict(seqlen=-1), ssd.SSD_ERR_INVALID_ARG),
    (dict(nheads=0), ssd.SSD_ERR_INVALID_ARG),
    (dict(headdim=32), ssd.SSD_ERR_UNSUPPORTED),
    (dict(dstate=48), ssd.SSD_ERR_UNSUPPORTED),
    (dict(chunk_size=100), ssd.SSD_ERR_UNSUPPORTED),
    (dict(chunk_size=32), ssd.SSD_ERR_UNSUPPORTED),
    (dict(bf16=False, dstate=256, headdim=128), ssd.SSD_ERR_UNSUPPORTED),
    (dict(dt_min=0.5, dt_max=0.1), ssd.SSD_ERR_INVALID_ARG),
    (dict(dt_min=float("nan")), ssd.SSD_ERR_INVALID_ARG),
    (dict(algo=7), ssd.SSD_ERR_INVALID_ARG),
])
def test_invalid_problems_are_rejected_on_the_host(kw, status):
    assert call(good(**kw), ws_bytes=1 << 30) == status


def test_other_host_rejections():
    p = good()
    assert call(p, prob_ptr=False) == ssd.SSD_ERR_INVALID_ARG
    q = good(); q.dtype = 7
    assert call(q) == ssd.SSD_ERR_INVALID_ARG
    q = good(); q.flags = 1 << 5
    assert call(q) == ssd.SSD_ERR_INVALID_ARG
    # C groups: 0 (same as B) or a divisor of H
    q = good(); q.ngroups_c = 3  # H = 4
    assert call(q) == ssd.SSD_ERR_INVALID_ARG
    q = good(); q.ngroups_c = -1
    assert call(q) == ssd.SSD_ERR_INVALID_ARG
    q = good(); q.ngroups_c = 4
    assert ssd.workspace_size(q) > 0
    assert call(p, x=None) == ssd.SSD_ERR_INVALID_ARG
    assert call(p, y=None) == ssd.SSD_ERR_INVALID_ARG
    # workspace missing, too small, misaligned
    assert call(p, ws=None) == ssd.SSD_ERR_WORKSPACE
    assert call(p, ws_bytes=ssd.workspace_size(p) - 256) == ssd.SSD_ERR_WORKSPACE
    assert call(p, ws=FAKE + 16) == ssd.SSD_ERR_INVALID_ARG
    # cu_seqlens requires batch == 1 and at least one sequence
    assert call(good(batch=2, nseqs=3), cu=FAKE) == ssd.SSD_ERR_INVALID_ARG
    assert call(good(batch=1, nseqs=0), cu=FAKE) == ssd.SSD_ERR_INVALID_ARG


def test_dt_cumsum_validation():
    lib = ssd.library()
    p = good(ngroups=3)
    assert lib.ssd_dt_cumsum(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None) == \
        ssd.SSD_ERR_INVALID_ARG
    p = good()
    assert lib.ssd_dt_cumsum(ctypes.byref(p), None, FAKE, None, FAKE, FAKE, None) == \
        ssd.SSD_ERR_INVALID_ARG


def test_step_validation():
    """The single-token step checks its problem on the host (seqlen 1, P 64/128,
    groups dividing heads, flags, clamp bounds, required pointers)."""
    lib = ssd.library()

    def step(p, **ptrs):
        args = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, bias=None, state=FAKE,
                    y=FAKE)
        args.update(ptrs)
        return lib.ssd_step(ctypes.byref(p), args["x"], args["dt"], args["A"], args["B"],
                            args["C"], args["D"], args["bias"], args["state"], args["y"], None)

    assert lib.ssd_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == \
        ssd.SSD_ERR_INVALID_ARG
    assert step(good(seqlen=2)) == ssd.SSD_ERR_INVALID_ARG
    assert step(good(seqlen=1, ngroups=3)) == ssd.SSD_ERR_INVALID_ARG
    assert step(good(seqlen=1, headdim=32)) == ssd.SSD_ERR_UNSUPPORTED
    q = good(seqlen=1); q.flags = 1 << 4
    assert step(q) == ssd.SSD_ERR_INVALID_ARG
    q = good(seqlen=1); q.dt_min, q.dt_max = 1.0, 0.5
    assert step(q) == ssd.SSD_ERR_INVALID_ARG
    for name in ("x", "dt", "A", "B", "C", "state", "y"):
        assert step(good(seqlen=1), **{name: None}) == ssd.SSD_ERR_INVALID_ARG, name
    # no rows: nothing to do, no pointer needed
    assert step(good(batch=0, seqlen=1), x=None, y=None, state=None) == ssd.SSD_OK


def test_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(1, 64, 2, 64)
    with pytest.raises(ValueError):
        ssd.fwd(x, torch.zeros(1, 64, 2), torch.zeros(2), torch.zeros(1, 64, 1, 16),
                torch.zeros(1, 64, 1, 16))


def test_bwd_workspace_size_rules():
    """ssd_bwd_workspace_size: zero for shapes the backward does not take (fp32
    with N P > 8192, bf16 with N P > 16384), positive otherwise (packed
    sequences included), and growing with the sequence length."""
    lib = ssd.library()
    size = lambda **kw: lib.ssd_bwd_workspace_size(ctypes.byref(ssd.make_problem(**kw)))  # noqa
    base = dict(batch=2, seqlen=1000, nheads=4, headdim=64, dstate=128, ngroups=1, chunk_size=256)
    assert size(**base) > 0
    assert size(**{**base, "seqlen": 2000}) > size(**base)
    assert size(**{**base, "bf16": False, "headdim": 128}) == 0
    assert size(**{**base, "bf16": False}) > 0
    assert size(**{**base, "headdim": 128, "dstate": 256}) == 0
    assert size(**{**base, "batch": 1, "nseqs": 3}) > 0  # packed sequences


def call_bwd(p, ws_bytes=None, cu=None, dy=FAKE, dx=FAKE, dA=FAKE, ws=FAKE):
    lib = ssd.library()
    if ws_bytes is None:
        ws_bytes = lib.ssd_bwd_workspace_size(ctypes.byref(p))
    # x dt A B C D dt_bias init cu dy dfinal | dx ddt dA dB dC dD ddt_bias dinit | ws bytes stream
    return lib.ssd_bwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, cu, dy,
                       None, dx, FAKE, dA, FAKE, FAKE, None, None, None, ws, ws_bytes, None)


def test_bwd_host_rejections():
    """ssd_bwd returns its error before enqueuing anything: unsupported shapes
    are UNSUPPORTED, missing tensors INVALID_ARG, a missing or short workspace
    WORKSPACE, a misaligned one INVALID_ARG.  Packed sequences with
    per-sequence states pass the checks up to the workspace."""
    p = good()
    assert call_bwd(p, cu=FAKE) == ssd.SSD_ERR_INVALID_ARG  # packed input needs batch 1
    v = good(batch=1, nseqs=3)
    lib = ssd.library()
    # packed sequences with initial states, final-state and initial-state
    # gradients: accepted (no workspace given, so nothing is enqueued)
    assert lib.ssd_bwd(ctypes.byref(v), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE,
                       FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None,
                       0, None) == ssd.SSD_ERR_WORKSPACE
    assert lib.ssd_bwd_workspace_size(ctypes.byref(v)) > lib.ssd_bwd_workspace_size(
        ctypes.byref(good(batch=1)))
    assert call_bwd(good(bf16=False, headdim=128, dstate=128)) == ssd.SSD_ERR_UNSUPPORTED
    assert call_bwd(good(dstate=256, headdim=128)) == ssd.SSD_ERR_UNSUPPORTED
    q = good(); q.ngroups_c = 3
    assert call_bwd(q, ws_bytes=1 << 30) == ssd.SSD_ERR_INVALID_ARG
    assert call_bwd(p, dy=None) == ssd.SSD_ERR_INVALID_ARG
    assert call_bwd(p, dx=None) == ssd.SSD_ERR_INVALID_ARG
    assert call_bwd(p, dA=None) == ssd.SSD_ERR_INVALID_ARG
    assert call_bwd(p, ws=None) == ssd.SSD_ERR_WORKSPACE
    need = ssd.library().ssd_bwd_workspace_size(ctypes.byref(p))
    assert call_bwd(p, ws_bytes=need - 256) == ssd.SSD_ERR_WORKSPACE
    assert call_bwd(p, ws=FAKE + 16) == ssd.SSD_ERR_INVALID_ARG


