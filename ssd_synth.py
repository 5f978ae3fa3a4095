"""Seeded synthetic inputs for the SSD forward pass.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no softplus, no exp, no cumulative sums).  Both the GPU
path's tests/benchmark and the CPU oracle consume what it produces.

The workloads are Mamba-2-shaped layers ("Transformers are SSMs": section 2.4
fixes head dims P in {64, 128}; section 7.1 shares B/C heads; section 8.3 packs
variable-length sequences; section 9.1 sweeps the state size N in {16, 64, 256};
appendix D.3 gives the 2.7B model d_model 2560, i.e. d_inner 5120 = 80 x 64).
The pages measure on datasets (the Pile, the LM evaluation suite, MQAR); these
seeded tensors stand in for them and reproduce none of their items.

Recipe (per workload k, numpy PCG64, seed 20240531 + k; sweep case (iL, iN) uses
20240531 + 300 + 10 iL + iN), drawn in this order:
  lengths  (varlen only) 64 draws rint(exp(U(ln 64, ln 8192))), packed in order
           and cut at 65536 tokens (the straddling sequence is shortened, later
           ones dropped)
  x        N(0, 1)                       (b, L, H, P)      float32 draw
  dt_raw   N(0, 1) - 4.6                 (b, L, H)         float32 draw
  A        -exp(U(0, ln 16))             (H,)              float64 -> float32
  B, C     N(0, 1/N)  (std 1/sqrt(N))    (b, L, G, N)      float32 draw
  D        N(0, 1)                       (H,)              float64 -> float32
  init     N(0, 1)   (sweep only)        (S, H, N, P)      float32 draw
dt is passed raw with the softplus flag and the clamp [1e-3, 0.1], so the
layer sees dt = clamp(softplus(N(0,1) - 4.6), 1e-3, 0.1).  For bf16 workloads
x, dt, B, C are rounded to bfloat16 (round to nearest even) and kept as float32
arrays holding exactly those bf16 values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

BASE_SEED = 20240531
DT_MIN, DT_MAX = 1e-3, 0.1
SWEEP_L = (512, 2048, 8192, 16384, 65536)
SWEEP_N = (16, 64, 128, 256)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str  # "f32" or "bf16"
    seed: int
    with_init: bool = False
    want_final: bool = True
    varlen: bool = False
    description: str = ""

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


def workloads() -> Dict[str, Workload]:
    w = {
        "tiny_f32": Workload("tiny_f32", 1, 256, 2, 64, 16, 1, 64, "f32", BASE_SEED + 0,
                             description="b1 L256 H2 P64 N16 G1 Q64 fp32, zero initial state"),
        "mamba2_130m": Workload("mamba2_130m", 8, 2048, 24, 64, 128, 1, 256, "bf16",
                                BASE_SEED + 1, want_final=False,
                                description="Mamba-2-130M-shaped layer: b8 L2048 H24 P64 N128 G1 Q256 bf16"),
        "mamba2_2p7b": Workload("mamba2_2p7b", 4, 4096, 80, 64, 128, 1, 256, "bf16",
                                BASE_SEED + 2, want_final=False,
                                description="Mamba-2-2.7B-shaped layer: b4 L4096 H80 P64 N128 G1 Q256 bf16"),
        "varlen_80h": Workload("varlen_80h", 1, 65536, 80, 64, 128, 8, 256, "bf16", BASE_SEED + 4,
                               varlen=True,
                               description="64 packed sequences, lengths log-uniform [64, 8192], "
                                           "cut at 65536 tokens, H80 P64 N128 G8 Q256 bf16"),
    }
    for iL, L in enumerate(SWEEP_L):
        for iN, N in enumerate(SWEEP_N):
            name = f"sweep_L{L}_N{N}"
            w[name] = Workload(name, 1, L, 32, 64, N, 1, 256, "bf16",
                               BASE_SEED + 300 + 10 * iL + iN, with_init=True,
                               description=f"sweep b1 H32 P64 L{L} N{N} Q256 bf16, random initial state")
    return w


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def varlen_lengths(rng: np.random.Generator, count: int = 64, lo: int = 64, hi: int = 8192,
                   total: int = 65536) -> List[int]:
    raw = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=count))).astype(np.int64)
    out, acc = [], 0
    for n in raw:
        if acc >= total:
            break
        n = int(min(n, total - acc))
        out.append(n)
        acc += n
    return out


@dataclass
class Inputs:
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: Optional[np.ndarray]
    dt_bias: Optional[np.ndarray] = None
    initial_states: Optional[np.ndarray] = None
    cu_seqlens: Optional[np.ndarray] = None
    chunk: int = 256
    dtype: str = "bf16"
    softplus: bool = True
    scales_input: bool = False
    dt_min: float = DT_MIN
    dt_max: float = DT_MAX
    want_final: bool = True
    meta: Dict = field(default_factory=dict)

    @property
    def nseqs(self) -> int:
        return (self.cu_seqlens.shape[0] - 1) if self.cu_seqlens is not None else self.x.shape[0]


def draw(rng: np.random.Generator, batch: int, seqlen: int, H: int, P: int, N: int, G: int,
         dtype: str, with_init: bool, nseqs: Optional[int] = None, Gc: Optional[int] = None):
    x = rng.standard_normal((batch, seqlen, H, P), dtype=np.float32)
    dt = rng.standard_normal((batch, seqlen, H), dtype=np.float32) - np.float32(4.6)
    A = (-np.exp(rng.uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    s = np.float32(1.0 / math.sqrt(N))
    B = rng.standard_normal((batch, seqlen, G, N), dtype=np.float32) * s
    C = rng.standard_normal((batch, seqlen, G if Gc is None else Gc, N), dtype=np.float32) * s
    D = rng.standard_normal(H).astype(np.float32)
    init = None
    if with_init:
        S = batch if nseqs is None else nseqs
        init = rng.standard_normal((S, H, N, P), dtype=np.float32)
    if dtype == "bf16":
        x, dt, B, C = (round_to_bf16(v) for v in (x, dt, B, C))
    return x, dt, A, B, C, D, init


def make(name: str) -> Inputs:
    """Inputs of one named workload (see workloads())."""
    w = workloads()[name]
    rng = np.random.default_rng(w.seed)
    cu = None
    meta = {"workload": w.name, "seed": w.seed, "description": w.description}
    if w.varlen:
        lengths = varlen_lengths(rng)
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        meta["lengths"] = lengths
        seqlen = int(cu[-1])
    else:
        seqlen = w.seqlen
    x, dt, A, B, C, D, init = draw(rng, w.batch, seqlen, w.nheads, w.headdim, w.dstate,
                                   w.ngroups, w.dtype, w.with_init,
                                   None if cu is None else len(cu) - 1)
    return Inputs(x, dt, A, B, C, D, None, init, cu, w.chunk, w.dtype, True, False, DT_MIN, DT_MAX,
                  w.want_final, meta)


def random_case(seed: int, batch: int, seqlen: int, H: int, P: int, N: int, G: int = 1,
                chunk: int = 64, dtype: str = "f32", with_init: bool = False,
                lengths: Optional[List[int]] = None, with_D: bool = True,
                Gc: Optional[int] = None) -> Inputs:
    """A seeded case of arbitrary shape with the workload distributions.

    With ``lengths`` the case is a packed varlen batch (batch must be 1 and
    sum(lengths) == seqlen); zero lengths are allowed.  ``Gc`` gives C its own
    group count (default: G, the B group count).
    """
    rng = np.random.default_rng(seed)
    cu = None
    nseqs = None
    if lengths is not None:
        assert batch == 1 and sum(lengths) == seqlen
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        nseqs = len(lengths)
    x, dt, A, B, C, D, init = draw(rng, batch, seqlen, H, P, N, G, dtype, with_init, nseqs, Gc)
    return Inputs(x, dt, A, B, C, D if with_D else None, None, init, cu, chunk, dtype, True, False,
                  DT_MIN, DT_MAX, True, {"seed": seed})


def random_grads(seed: int, inp: Inputs, with_dfinal: bool = True):
    """Seeded upstream gradients for a case: dy like y (standard normal, rounded
    to bf16 for bf16 storage) and dfinal like the final states (standard
    normal, float32) or None."""
    rng = np.random.default_rng(seed)
    b, L, H, P = inp.x.shape
    N = inp.B.shape[3]
    dy = rng.standard_normal((b, L, H, P), dtype=np.float32)
    if inp.dtype == "bf16":
        dy = round_to_bf16(dy)
    dfin = rng.standard_normal((inp.nseqs, H, N, P), dtype=np.float32) if with_dfinal else None
    return dy, dfin


def large_case_device(seed: int, batch: int, seqlen: int, H: int, P: int, N: int,
                      device: str = "cuda"):
    """A bf16 case too large to draw on the host in reasonable time (x and y
    with more than 2^31 elements), drawn on the device with torch's seeded
    counter-based generator, with the workload distributions of draw():
    x ~ N(0, 1), dt_raw ~ N(0, 1) - 4.6, A = -exp(U(0, ln 16)), B, C ~ N(0, 1/N),
    D ~ N(0, 1); one B/C group.  Returns a dict of device tensors (x, dt, B, C in
    bf16; A, D in fp32)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    bf = torch.bfloat16
    x = torch.empty((batch, seqlen, H, P), dtype=bf, device=device)
    # drawn in row slices so that the float32 draw never holds the whole tensor
    for b in range(batch):
        x[b].copy_(torch.randn((seqlen, H, P), generator=g, device=device))
    dt = (torch.randn((batch, seqlen, H), generator=g, device=device) - 4.6).to(bf)
    A = -torch.exp(torch.rand((H,), generator=g, device=device, dtype=torch.float64) *
                   math.log(16.0)).float()
    s = 1.0 / math.sqrt(N)
    B = (torch.randn((batch, seqlen, 1, N), generator=g, device=device) * s).to(bf)
    C = (torch.randn((batch, seqlen, 1, N), generator=g, device=device) * s).to(bf)
    D = torch.randn((H,), generator=g, device=device)
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D)


def host_subset(dev: dict, heads: List[int], chunk: int = 256) -> Inputs:
    """The heads `heads` of a device case as host Inputs (the bf16 values held
    exactly in float32 arrays), every row, for the oracle."""
    import torch

    idx = torch.tensor(heads, device=dev["x"].device)
    f = lambda t: t.float().cpu().numpy()
    x = f(dev["x"].index_select(2, idx))
    dt = f(dev["dt"].index_select(2, idx))
    A = dev["A"].cpu().numpy()[heads]
    D = dev["D"].cpu().numpy()[heads]
    return Inputs(x, dt, A, f(dev["B"]), f(dev["C"]), D, None, None, None, chunk, "bf16", True,
                  False, DT_MIN, DT_MAX, True, {"heads": list(heads)})


def large_grad_device(seed: int, like, device: str = "cuda"):
    """A seeded tensor ~ N(0, 1) (an upstream gradient, a state) shaped like the device tensor
    `like` (drawn per row on the device, stored in its dtype)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dy = torch.empty_like(like)
    for b in range(like.shape[0]):
        dy[b].copy_(torch.randn(like.shape[1:], generator=g, device=device))
    return dy
