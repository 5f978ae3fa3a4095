"""MI355X-native chunked SSD (state space duality) forward pass.

Python binding of ``libssd.so`` (HIP kernels for gfx950 behind the C ABI in
``include/ssd.h``).  This module only marshals arguments: it checks tensor
devices, dtypes and shapes, allocates outputs and workspace with torch, and
calls the C entry points of the same names.  Every step of the computation runs
in the library's kernels; there is no fallback of any kind.  The first call
fails loudly (ImportError) if the library has not been built
(``python -m ssd_scan_amd.build``).

The operation ("Transformers are SSMs", section 2.4 scalar-times-identity SSM,
section 6 block decomposition, section 8.3 variable length): per head h with
B/C group g = h // (H // G),

    S_t = exp(dt'_t A_h) S_{t-1} + B_t x_t^T,    y_t = C_t^T S_t + D_h x_t,

with dt'_t = clamp(softplus(dt_t + dt_bias_h), dt_min, dt_max) (softplus optional).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libssd.so")

SSD_OK, SSD_ERR_INVALID_ARG, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_HIP = range(5)
SSD_DTYPE_F32, SSD_DTYPE_BF16 = 0, 1
SSD_DT_SOFTPLUS, SSD_DT_SCALES_INPUT = 1, 2
ALGOS = {"auto": 0, "chunked": 1, "fused": 2, "stream": 3}


class SsdProblem(ctypes.Structure):
    """Mirror of ``ssd_problem`` in include/ssd.h."""

    _fields_ = [
        ("batch", ctypes.c_int64),
        ("seqlen", ctypes.c_int64),
        ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64),
        ("dstate", ctypes.c_int64),
        ("ngroups", ctypes.c_int64),
        ("chunk_size", ctypes.c_int64),
        ("nseqs", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("dt_min", ctypes.c_float),
        ("dt_max", ctypes.c_float),
        ("algo", ctypes.c_int32),
        ("ngroups_c", ctypes.c_int32),
    ]


class SsdError(RuntimeError):
    def __init__(self, status: int, what: str = "ssd_fwd"):
        self.status = status
        super().__init__(f"{what} failed: {status_string(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is missing: build it with `python -m ssd_scan_amd.build`")
    lib = ctypes.CDLL(LIBRARY)
    P = ctypes.c_void_p
    pp = ctypes.POINTER(SsdProblem)
    lib.ssd_workspace_size.restype = ctypes.c_size_t
    lib.ssd_workspace_size.argtypes = [pp]
    lib.ssd_fwd_noalloc.restype = ctypes.c_int
    lib.ssd_fwd_noalloc.argtypes = [pp] + [P] * 11 + [P]
    lib.ssd_fwd.restype = ctypes.c_int
    lib.ssd_fwd.argtypes = [pp, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.ssd_fwd_events.restype = ctypes.c_int
    lib.ssd_fwd_events.argtypes = [pp, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P,
                                   ctypes.POINTER(ctypes.c_void_p),
                                   ctypes.POINTER(ctypes.c_char_p), ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_int)]
    lib.ssd_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ssd_bwd_workspace_size.argtypes = [pp]
    bwd_args = [pp] + [P] * 20 + [ctypes.c_size_t, P]
    lib.ssd_bwd.restype = ctypes.c_int
    lib.ssd_bwd.argtypes = bwd_args
    lib.ssd_bwd_events.restype = ctypes.c_int
    lib.ssd_bwd_events.argtypes = bwd_args + [P, P, ctypes.c_int, P]
    lib.ssd_dt_cumsum.restype = ctypes.c_int
    lib.ssd_dt_cumsum.argtypes = [pp, P, P, P, P, P, P]
    lib.ssd_step.restype = ctypes.c_int
    lib.ssd_step.argtypes = [pp, P, P, P, P, P, P, P, P, P, P]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_version.restype = ctypes.c_char_p
    lib.ssd_version.argtypes = []
    return lib


_lib: Optional[ctypes.CDLL] = None


def library() -> ctypes.CDLL:
    """The loaded libssd.so (loaded on first use; raises ImportError if it is not built)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def status_string(status: int) -> str:
    return library().ssd_status_string(int(status)).decode()


def version() -> str:
    return library().ssd_version().decode()


def make_problem(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, *, bf16=True,
                 nseqs=0, softplus=True, scales_input=False, dt_min=0.0, dt_max=math.inf,
                 algo="auto", ngroups_c=0) -> SsdProblem:
    p = SsdProblem()
    p.batch, p.seqlen, p.nheads, p.headdim = batch, seqlen, nheads, headdim
    p.dstate, p.ngroups, p.chunk_size, p.nseqs = dstate, ngroups, chunk_size, nseqs
    p.dtype = SSD_DTYPE_BF16 if bf16 else SSD_DTYPE_F32
    p.flags = (SSD_DT_SOFTPLUS if softplus else 0) | (SSD_DT_SCALES_INPUT if scales_input else 0)
    p.dt_min, p.dt_max = float(dt_min), float(dt_max)
    p.algo = ALGOS[algo] if isinstance(algo, str) else int(algo)
    p.ngroups_c = ngroups_c
    return p


def workspace_size(problem: SsdProblem) -> int:
    return int(library().ssd_workspace_size(ctypes.byref(problem)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch

    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(x, dt, A, B, C, D=None, dt_bias=None, initial_states=None, cu_seqlens=None, *,
        chunk_size: int = 256, softplus: bool = True, scales_input: bool = False,
        dt_min: float = 0.0, dt_max: float = math.inf, algo="auto",
        return_final_states: bool = False, out=None, final_states=None, workspace=None,
        stream=None, library_scratch: bool = False):
    """Chunked SSD forward on the GPU.

    x (b, L, H, P), dt (b, L, H), B (b, L, G, N), C (b, L, Gc, N) in float32 or
    bfloat16 (all the same; G and Gc divide H and may differ); A, D, dt_bias (H,)
    float32; initial_states (S, H, N, P) float32 with
    S = b, or S = len(cu_seqlens) - 1 for packed sequences (then b == 1);
    cu_seqlens int32.  Returns y, or (y, final_states) with return_final_states.
    library_scratch=True calls ssd_fwd_noalloc (the library's own device
    scratch buffer, no workspace; SsdError with SSD_ERR_WORKSPACE when the
    problem needs more than SSD_NOALLOC_SCRATCH_BYTES).
    """
    import torch

    if x.dim() != 4:
        raise ValueError("x must be (batch, seqlen, heads, headdim)")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    Gc = C.shape[2] if C.dim() == 4 else G
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_scan_amd runs on the GPU only; x is on " + str(dev))
    dtype = x.dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    nseqs = 0
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
        nseqs = cu_seqlens.shape[0] - 1
    S = nseqs if cu_seqlens is not None else b
    _check(x, "x", (b, L, H, P), dtype, dev)
    _check(dt, "dt", (b, L, H), dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(B, "B", (b, L, G, N), dtype, dev)
    _check(C, "C", (b, L, Gc, N), dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(initial_states, "initial_states", (S, H, N, P), torch.float32, dev)
    prob = make_problem(b, L, H, P, N, G, chunk_size, bf16=dtype == torch.bfloat16, nseqs=nseqs,
                        softplus=softplus, scales_input=scales_input, dt_min=dt_min,
                        dt_max=dt_max, algo=algo, ngroups_c=0 if Gc == G else Gc)
    y = out if out is not None else torch.empty_like(x)
    _check(y, "out", (b, L, H, P), dtype, dev)
    fin = None
    if return_final_states or final_states is not None:
        fin = final_states if final_states is not None else torch.empty(
            (S, H, N, P), dtype=torch.float32, device=dev)
        _check(fin, "final_states", (S, H, N, P), torch.float32, dev)
    if library_scratch:
        st = library().ssd_fwd_noalloc(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                       _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(initial_states),
                                       _ptr(cu_seqlens), _ptr(y), _ptr(fin), _stream(stream))
        if st != SSD_OK:
            raise SsdError(st, "ssd_fwd_noalloc")
        return (y, fin) if (return_final_states or final_states is not None) else y
    need = workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = library().ssd_fwd(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                      _ptr(dt_bias), _ptr(initial_states), _ptr(cu_seqlens), _ptr(y), _ptr(fin),
                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                      _stream(stream))
    if st != SSD_OK:
        raise SsdError(st)
    return (y, fin) if (return_final_states or final_states is not None) else y


def bwd_workspace_size(problem: SsdProblem) -> int:
    return int(library().ssd_bwd_workspace_size(ctypes.byref(problem)))


def bwd(x, dt, A, B, C, dy, D=None, dt_bias=None, initial_states=None, d_final_states=None,
        cu_seqlens=None, *, softplus: bool = True, scales_input: bool = False,
        dt_min: float = 0.0, dt_max: float = math.inf, workspace=None, stream=None, events=None):
    """Gradients of the chunked SSD layer on the GPU.

    Inputs as for ``fwd`` plus dy (b, L, H, P) in the storage dtype and
    d_final_states (S, H, N, P) float32 (zero when None), S = b, or S =
    len(cu_seqlens) - 1 for packed sequences (b == 1; initial_states is then
    (S, H, N, P) as well).  Returns a dict: dx, ddt, dB, dC in the storage
    dtype; dA, dD, ddt_bias (H,) and dinit (S, H, N, P) in float32.  With ``events`` (a list of torch.cuda.Event with
    enable_timing), events are recorded before each kernel and after the last;
    the dict then also holds "kernels", the name of each interval.
    """
    import torch

    if x.dim() != 4:
        raise ValueError("x must be (batch, seqlen, heads, headdim)")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    Gc = C.shape[2] if C.dim() == 4 else G
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_scan_amd runs on the GPU only; x is on " + str(dev))
    dtype = x.dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _check(x, "x", (b, L, H, P), dtype, dev)
    _check(dt, "dt", (b, L, H), dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(B, "B", (b, L, G, N), dtype, dev)
    _check(C, "C", (b, L, Gc, N), dtype, dev)
    _check(dy, "dy", (b, L, H, P), dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    nseqs = 0
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (cu_seqlens.shape[0],), torch.int32, dev)
        nseqs = cu_seqlens.shape[0] - 1
    S = nseqs if cu_seqlens is not None else b
    _check(initial_states, "initial_states", (S, H, N, P), torch.float32, dev)
    _check(d_final_states, "d_final_states", (S, H, N, P), torch.float32, dev)
    prob = make_problem(b, L, H, P, N, G, 64, bf16=dtype == torch.bfloat16, nseqs=nseqs,
                        softplus=softplus, scales_input=scales_input, dt_min=dt_min,
                        dt_max=dt_max, ngroups_c=0 if Gc == G else Gc)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt), "dB": torch.empty_like(B),
           "dC": torch.empty_like(C), "dA": torch.empty(H, **f32), "dD": torch.empty(H, **f32),
           "ddt_bias": torch.empty(H, **f32),
           "dinit": torch.empty((S, H, N, P), **f32)}
    need = bwd_workspace_size(prob)
    if need == 0 and b * L > 0:
        raise SsdError(SSD_ERR_UNSUPPORTED, "ssd_bwd")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = [ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(dt_bias), _ptr(initial_states), _ptr(cu_seqlens), _ptr(dy), _ptr(d_final_states),
            _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
            _ptr(out["dD"]), _ptr(out["ddt_bias"]), _ptr(out["dinit"]), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    if events is None:
        st = library().ssd_bwd(*args)
    else:
        n = len(events)
        names = (ctypes.c_char_p * n)()
        count = ctypes.c_int(0)
        for e in events:  # create the underlying HIP events before handing them over
            e.record()
        handles = (ctypes.c_void_p * n)(*[ctypes.c_void_p(e.cuda_event) for e in events])
        st = library().ssd_bwd_events(*args, handles, names, n, ctypes.byref(count))
        out["kernels"] = [names[i].decode() for i in range(count.value)]
    if st != SSD_OK:
        raise SsdError(st, "ssd_bwd")
    return out


def step(x, dt, A, B, C, state, D=None, dt_bias=None, *, softplus: bool = True,
         scales_input: bool = False, dt_min: float = 0.0, dt_max: float = math.inf, out=None,
         stream=None):
    """One token of the recurrence (decode) for each row, on the GPU.

    x (b, H, P), dt (b, H), B (b, G, N), C (b, Gc, N) in float32 or bfloat16 (all the same);
    A, D, dt_bias (H,) float32; state (b, H, N, P) float32, updated in place.
    Returns y (b, H, P).
    """
    import torch

    if x.dim() != 3:
        raise ValueError("x must be (batch, heads, headdim)")
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    Gc = C.shape[1] if C.dim() == 3 else G
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_scan_amd runs on the GPU only; x is on " + str(dev))
    dtype = x.dtype
    if dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _check(x, "x", (b, H, P), dtype, dev)
    _check(dt, "dt", (b, H), dtype, dev)
    _check(A, "A", (H,), torch.float32, dev)
    _check(B, "B", (b, G, N), dtype, dev)
    _check(C, "C", (b, Gc, N), dtype, dev)
    _check(D, "D", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    _check(state, "state", (b, H, N, P), torch.float32, dev)
    prob = make_problem(b, 1, H, P, N, G, 64, bf16=dtype == torch.bfloat16, softplus=softplus,
                        scales_input=scales_input, dt_min=dt_min, dt_max=dt_max,
                        ngroups_c=0 if Gc == G else Gc)
    y = out if out is not None else torch.empty_like(x)
    _check(y, "out", (b, H, P), dtype, dev)
    st = library().ssd_step(ctypes.byref(prob), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                            _ptr(D), _ptr(dt_bias), _ptr(state), _ptr(y), _stream(stream))
    if st != SSD_OK:
        raise SsdError(st)
    return y


def dt_cumsum(dt, A, dt_bias=None, *, chunk_size: int = 256, softplus: bool = True,
              dt_min: float = 0.0, dt_max: float = math.inf, stream=None):
    """dt' and the per-chunk inclusive prefix sums of dt' A, each (b, H, nchunks, Q) float32."""
    import torch

    b, L, H = dt.shape
    dev = dt.device
    _check(A, "A", (H,), torch.float32, dev)
    _check(dt_bias, "dt_bias", (H,), torch.float32, dev)
    nc = (L + chunk_size - 1) // chunk_size
    prob = make_problem(b, L, H, 64, 16, 1, chunk_size, bf16=dt.dtype == torch.bfloat16,
                        softplus=softplus, dt_min=dt_min, dt_max=dt_max)
    dto = torch.empty((b, H, nc, chunk_size), dtype=torch.float32, device=dev)
    cso = torch.empty_like(dto)
    st = library().ssd_dt_cumsum(ctypes.byref(prob), _ptr(dt.contiguous()), _ptr(A), _ptr(dt_bias),
                            _ptr(dto), _ptr(cso), _stream(stream))
    if st != SSD_OK:
        raise SsdError(st, "ssd_dt_cumsum")
    return dto, cso


def _autograd_function():
    import torch

    class _SsdScan(torch.autograd.Function):
        """ssd_fwd forward, ssd_bwd backward (argument marshalling only)."""

        @staticmethod
        def forward(ctx, x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens, opts):
            y, fin = fwd(x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens,
                         return_final_states=True, **opts)
            ctx.save_for_backward(x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens)
            ctx.opts = {k: v for k, v in opts.items() if k not in ("chunk_size", "algo")}
            return y, fin

        @staticmethod
        def backward(ctx, dy, dfin=None):
            x, dt, A, B, C, D, dt_bias, init, cu = ctx.saved_tensors
            g = bwd(x, dt, A, B, C, dy.contiguous(), D, dt_bias, init,
                    None if dfin is None else dfin.contiguous(), cu, **ctx.opts)
            return (g["dx"], g["ddt"], g["dA"], g["dB"], g["dC"],
                    g["dD"] if D is not None else None,
                    g["ddt_bias"] if dt_bias is not None else None,
                    g["dinit"] if init is not None else None, None, None)

    return _SsdScan


_FN = None


def ssd_scan(x, dt, A, B, C, D=None, dt_bias=None, initial_states=None, cu_seqlens=None, *,
             chunk_size: int = 256, softplus: bool = True, scales_input: bool = False,
             dt_min: float = 0.0, dt_max: float = math.inf):
    """Differentiable SSD layer for PyTorch autograd: the forward pass runs
    ``ssd_fwd`` and the backward pass ``ssd_bwd``.  Returns (y, final_states),
    final_states (S, H, N, P) with S = b, or S = len(cu_seqlens) - 1 for
    packed sequences; the same shapes and options as ``fwd``."""
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    opts = dict(chunk_size=chunk_size, softplus=softplus, scales_input=scales_input,
                dt_min=dt_min, dt_max=dt_max)
    return _FN.apply(x, dt, A, B, C, D, dt_bias, initial_states, cu_seqlens, opts)


__all__ = ["fwd", "bwd", "step", "ssd_scan", "dt_cumsum", "workspace_size",
           "bwd_workspace_size", "make_problem", "status_string", "version", "SsdProblem",
           "SsdError", "library", "LIBRARY"]
