"""fp64 CPU oracle for the SSD forward pass and its gradients.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or build anything in this
package.  The product path (``ssd_scan_amd``) never touches it, and this package
imports nothing from the product path.

The oracle is the token-by-token recurrence written in ``ssd_ref.c`` (see that
file's header for the definition and the passages it follows: "Transformers
are SSMs", section 3.4.1 linear mode, section 3.2.2 scalar recurrence, section
2.4 scalar-times-identity transition, section 8.3 variable length, section 8.2
state hand-off).  This module only compiles it with gcc and marshals numpy
arrays through ctypes.

Pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_pins.py`` (quadratic
form by brute force, a=1 prefix sums, a=0 diagonal, x=0 cumulative products,
linearity, chunk-size invariance of the block decomposition, varlen = separate
runs, state hand-off, group broadcast, skip term, dt preprocessing, and for the
single-token step its a=0 / a=1 / x=0 closed forms and chaining; for the
backward pass central differences of the forward oracle and reverse-mode
differentiation of the quadratic (matrix) form in PyTorch) and by the
planted-mistake tests in ``tests/test_oracle_mutants.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssd_ref.c")
LIBRARY = os.path.join(_HERE, "libssd_ref.so")

FLAG_SOFTPLUS = 1
FLAG_SCALES_INPUT = 2


def compile_oracle(source: str = SOURCE, output: str = LIBRARY, extra: Sequence[str] = ()) -> str:
    """Compile the C oracle into a shared library with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra, source, "-o",
           output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


def build() -> str:
    return compile_oracle()


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.ssd_ref_fwd.restype = ctypes.c_int
    lib.ssd_ref_fwd.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, p,  # shapes, cu_seqlens
                                p, p, p, p, p, p, p, p,  # x dt A B C D dt_bias init
                                ctypes.c_uint, ctypes.c_double, ctypes.c_double,
                                i64, p, p, p]
    lib.ssd_ref_bwd.restype = ctypes.c_int
    lib.ssd_ref_bwd.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64, p,  # shapes, cu_seqlens
                                p, p, p, p, p, p, p, p,  # x dt A B C D dt_bias init
                                ctypes.c_uint, ctypes.c_double, ctypes.c_double,
                                p, p,  # dy dfinal
                                p, p, p, p, p, p, p, p]  # dx ddt dA dB dC dD ddt_bias dinit
    lib.ssd_ref_num_threads.restype = ctypes.c_int
    lib.ssd_ref_num_threads.argtypes = []
    return lib


_LIB: Optional[ctypes.CDLL] = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the oracle library, compiling it first when it is missing or stale."""
    global _LIB
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _LIB is None:
        if (not os.path.exists(LIBRARY)
                or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        _LIB = _bind(ctypes.CDLL(LIBRARY))
    return _LIB


def num_threads(lib: Optional[ctypes.CDLL] = None) -> int:
    return int((lib or load()).ssd_ref_num_threads())


def _f32(a, name):
    if a is None:
        return None
    a = np.asarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"oracle input {name} must be float32 (got {a.dtype}); "
                        "widen bf16 values to float32 before the call")
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def ssd_ref(x, dt, A, B, C, D=None, dt_bias=None, initial_states=None, cu_seqlens=None, *,
            softplus: bool = False, scales_input: bool = False, dt_min: float = 0.0,
            dt_max: float = float("inf"), pairs=None, want_final: bool = True,
            lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Run the oracle.

    Shapes: x (b, L, H, P), dt (b, L, H), A (H), B (b, L, G, N), C (b, L, Gc, N) (G and
    Gc dividing H, possibly different), D/dt_bias (H),
    initial_states (S, H, N, P) with S = b, or S = nseqs when cu_seqlens (int32,
    nseqs+1) is given (then b must be 1).  All float inputs float32.

    Returns (y, final_states) in float64; final_states is None unless want_final.
    With ``pairs`` (iterable of (sequence, head)), only those streams are computed
    and the rest of y is NaN.
    """
    lib = lib or load()
    x, dt, A, B, C = (_f32(v, n) for v, n in ((x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C")))
    D, dt_bias, init = _f32(D, "D"), _f32(dt_bias, "dt_bias"), _f32(initial_states, "init")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    Gc = C.shape[2]
    if (dt.shape != (b, L, H) or A.shape != (H,) or B.shape != (b, L, G, N)
            or C.shape != (b, L, Gc, N)):
        raise ValueError("inconsistent shapes")
    cu = None
    nseqs = b
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        nseqs = cu.shape[0] - 1
    if init is not None and init.shape != (nseqs, H, N, P):
        raise ValueError("initial_states shape")
    pr = None
    n_pairs = 0
    if pairs is not None:
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        n_pairs = pr.shape[0]
    flags = (FLAG_SOFTPLUS if softplus else 0) | (FLAG_SCALES_INPUT if scales_input else 0)
    y = np.full((b, L, H, P), np.nan) if pairs is not None else np.empty((b, L, H, P))
    fin = np.full((nseqs, H, N, P), np.nan) if want_final else None
    rc = lib.ssd_ref_fwd(b, L, H, P, N, G, Gc, nseqs, _ptr(cu), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                         _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(init), flags, float(dt_min),
                         float(dt_max), n_pairs, _ptr(pr), _ptr(y), _ptr(fin))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return y, fin


def ssd_ref_step(x, dt, A, B, C, D=None, dt_bias=None, state=None, *, softplus: bool = False,
                 scales_input: bool = False, dt_min: float = 0.0, dt_max: float = float("inf"),
                 lib: Optional[ctypes.CDLL] = None) -> Tuple[np.ndarray, np.ndarray]:
    """The single-token (decode) step: one token of the recurrence for each of
    the b rows, from ``state`` (zero when None).

    Shapes: x (b, H, P), dt (b, H), A (H), B/C (b, G, N), D/dt_bias (H), state
    (b, H, N, P), all float32.  Returns (y (b, H, P), new state (b, H, N, P)) in
    float64.  This is the oracle above run over a one-token sequence (linear
    mode, section 3.4.1, one step); it adds no arithmetic of its own.
    """
    x, dt, B, C = (np.asarray(v)[:, None] for v in (x, dt, B, C))
    y, fin = ssd_ref(x, dt, A, B, C, D, dt_bias, state, softplus=softplus,
                     scales_input=scales_input, dt_min=dt_min, dt_max=dt_max, lib=lib)
    return y[:, 0], fin


def ssd_ref_bwd(x, dt, A, B, C, dy, D=None, dt_bias=None, initial_states=None, cu_seqlens=None,
                d_final_states=None, *, softplus: bool = False, scales_input: bool = False,
                dt_min: float = 0.0, dt_max: float = float("inf"), want_dinit: bool = True,
                lib: Optional[ctypes.CDLL] = None) -> dict:
    """Gradients of the layer for upstream gradients dy (like y) and
    d_final_states (like the final states; zero when None), by reverse-mode
    differentiation of the token recurrence (``ssd_ref_bwd`` in ssd_ref.c).

    Inputs as for ``ssd_ref`` plus dy (b, L, H, P) float32.  Returns a dict of
    float64 arrays: dx, ddt, dA, dB, dC, dD, ddt_bias and dinit (None unless
    want_dinit).  dD and ddt_bias are the gradients with respect to D and
    dt_bias also when those are None (taken as zero).
    """
    lib = lib or load()
    x, dt, A, B, C = (_f32(v, n) for v, n in ((x, "x"), (dt, "dt"), (A, "A"), (B, "B"), (C, "C")))
    D, dt_bias, init = _f32(D, "D"), _f32(dt_bias, "dt_bias"), _f32(initial_states, "init")
    dy, dfin = _f32(dy, "dy"), _f32(d_final_states, "d_final_states")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    Gc = C.shape[2]
    if (dt.shape != (b, L, H) or A.shape != (H,) or B.shape != (b, L, G, N)
            or C.shape != (b, L, Gc, N) or dy.shape != x.shape):
        raise ValueError("inconsistent shapes")
    cu = None
    nseqs = b
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        nseqs = cu.shape[0] - 1
    for v, nm in ((init, "initial_states"), (dfin, "d_final_states")):
        if v is not None and v.shape != (nseqs, H, N, P):
            raise ValueError(nm + " shape")
    flags = (FLAG_SOFTPLUS if softplus else 0) | (FLAG_SCALES_INPUT if scales_input else 0)
    out = {"dx": np.empty((b, L, H, P)), "ddt": np.empty((b, L, H)), "dA": np.empty(H),
           "dB": np.empty((b, L, G, N)), "dC": np.empty((b, L, Gc, N)), "dD": np.empty(H),
           "ddt_bias": np.empty(H), "dinit": np.empty((nseqs, H, N, P)) if want_dinit else None}
    rc = lib.ssd_ref_bwd(b, L, H, P, N, G, Gc, nseqs, _ptr(cu), _ptr(x), _ptr(dt), _ptr(A),
                         _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(init), flags,
                         float(dt_min), float(dt_max), _ptr(dy), _ptr(dfin),
                         *(_ptr(out[k]) for k in ("dx", "ddt", "dA", "dB", "dC", "dD",
                                                  "ddt_bias", "dinit")))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out
