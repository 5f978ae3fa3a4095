"""Independent fp64 formulations used to pin the oracle (tests only).

None of these share code with ``oracle/`` or with the GPU path.  Each is a
different way of writing the same layer that "Transformers are SSMs" says
must agree with the recurrence:

* ``quadratic_form``: the layer as one lower-triangular matrix y = M x
  (section 3.1 matrix transformation form, section 3.3 SSMs are semiseparable
  matrices, section 5.1/5.3 the quadratic dual form).  The decay products are
  built by repeated multiplication, not from logarithms.
* ``chunked_form``: the block decomposition of section 6 (diagonal blocks by
  the quadratic form with zero initial state, section 6.1; right factors to
  chunk states, a scalar scan across chunks, left factors from the incoming
  state, section 6.2), for any chunk length including 1 (the fully recurrent
  special case of appendix B.3.3) and T.
* ``dt_effective``: dt preprocessing written with numpy's logaddexp (softplus
  is log(1 + e^v) = logaddexp(0, v)) and clip.
"""
from __future__ import annotations

import numpy as np


def dt_effective(dt_raw, dt_bias=None, softplus=True, dt_min=0.0, dt_max=np.inf):
    v = np.asarray(dt_raw, dtype=np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, dtype=np.float64)
    if softplus:
        v = np.logaddexp(0.0, v)
    return np.clip(v, dt_min, dt_max)


def _streams(b, L, cu):
    if cu is None:
        return [(s, s, 0, L) for s in range(b)]  # (seq, batch row, start, stop)
    return [(s, 0, int(cu[s]), int(cu[s + 1])) for s in range(len(cu) - 1)]


def quadratic_form(x, dt, A, B, C, D=None, dt_bias=None, init=None, cu=None, softplus=True,
                   scales_input=False, dt_min=0.0, dt_max=np.inf):
    """y = M x + (init term) + D x, with M[t,u] = (C_t . B_u) a_{u+1} ... a_t for u <= t."""
    x = np.asarray(x, np.float64)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dte = dt_effective(dt, dt_bias, softplus, dt_min, dt_max)  # (b, L, H)
    y = np.zeros_like(x)
    nseq = b if cu is None else len(cu) - 1
    fin = np.zeros((nseq, H, N, P))
    for s, row, t0, t1 in _streams(b, L, cu):
        T = t1 - t0
        for h in range(H):
            g, gc = h // (H // G), h // (H // C.shape[2])
            a = np.exp(dte[row, t0:t1, h] * float(A[h]))
            Bs = np.asarray(B[row, t0:t1, g, :], np.float64)
            Cs = np.asarray(C[row, t0:t1, gc, :], np.float64)
            xs = x[row, t0:t1, h, :]
            scale = dte[row, t0:t1, h] if scales_input else np.ones(T)
            # decay[t, u] = prod_{k=u+1..t} a_k  (u <= t), built row by row.
            decay = np.zeros((T, T))
            for t in range(T):
                if t > 0:
                    decay[t, :t] = decay[t - 1, :t] * a[t]
                decay[t, t] = 1.0
            M = (Cs @ Bs.T) * decay * scale[None, :]
            ys = M @ xs
            # prod_{k=0..t} a_k applied to the initial state
            pre = np.cumprod(a) if T else a
            if init is not None:
                S0 = np.asarray(init[s, h], np.float64)
                ys = ys + (pre[:, None] * (Cs @ S0))
            if D is not None:
                ys = ys + float(D[h]) * xs
            y[row, t0:t1, h, :] = ys
            # final state = sum_u (prod_{k=u+1..T-1} a_k) B_u x_u^T + prod(a) init
            if T:
                w = decay[T - 1, :] * scale
                Sf = (Bs * w[:, None]).T @ xs
                if init is not None:
                    Sf = Sf + pre[-1] * np.asarray(init[s, h], np.float64)
            else:
                Sf = np.asarray(init[s, h], np.float64) if init is not None else np.zeros((N, P))
            fin[s, h] = Sf
    return y, fin


def chunked_form(x, dt, A, B, C, Q, D=None, dt_bias=None, init=None, cu=None, softplus=True,
                 scales_input=False, dt_min=0.0, dt_max=np.inf):
    """Block decomposition with chunk length Q (the last chunk of a stream may be shorter)."""
    x = np.asarray(x, np.float64)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dte = dt_effective(dt, dt_bias, softplus, dt_min, dt_max)
    y = np.zeros_like(x)
    nseq = b if cu is None else len(cu) - 1
    fin = np.zeros((nseq, H, N, P))
    for s, row, t0, t1 in _streams(b, L, cu):
        for h in range(H):
            g, gc = h // (H // G), h // (H // C.shape[2])
            state = (np.asarray(init[s, h], np.float64) if init is not None else np.zeros((N, P)))
            for c0 in range(t0, t1, Q):
                c1 = min(c0 + Q, t1)
                la = dte[row, c0:c1, h] * float(A[h])  # log decay
                cs = np.cumsum(la)  # inclusive segment sums from chunk start
                Bc = np.asarray(B[row, c0:c1, g, :], np.float64)
                Cc = np.asarray(C[row, c0:c1, gc, :], np.float64)
                xc = x[row, c0:c1, h, :]
                if scales_input:
                    xc_in = xc * dte[row, c0:c1, h][:, None]
                else:
                    xc_in = xc
                # diagonal block: (L o C B^T) X with L[i,j] = exp(cs_i - cs_j), j <= i
                seg = cs[:, None] - cs[None, :]
                causal = np.tril(np.ones(seg.shape, dtype=bool))
                Lm = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
                y_diag = (Lm * (Cc @ Bc.T)) @ xc_in
                # left factor: contribution of the incoming state
                y_off = np.exp(cs)[:, None] * (Cc @ state)
                yc = y_diag + y_off
                if D is not None:
                    yc = yc + float(D[h]) * xc
                y[row, c0:c1, h, :] = yc
                # right factor: chunk state from zero, then the scalar scan step
                w = np.exp(cs[-1] - cs)
                chunk_state = (Bc * w[:, None]).T @ xc_in
                state = np.exp(cs[-1]) * state + chunk_state
            fin[s, h] = state
    return y, fin


def rel_err(got, ref):
    """max_i |got_i - ref_i| / max(|ref_i|, rms(ref)) (0 for empty arrays)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rms if rms > 0 else 1e-300)
    return float(np.max(np.abs(got - ref) / den))
