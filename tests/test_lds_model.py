"""CPU model of the transposing LDS load (ds_read_b64_tr_b16) as the kernels
use it, checked for every tile kind they hand it: each lane's byte address is
8-byte aligned and inside the tile, and the 16-lane exchange gives every lane
the elements the plain per-lane reads would (lane (g, i) element e =
T[k0 + 4g + e][r0 + i]).

The exchange (per 16-lane group): source lane 4s + q supplies the 4 elements
at its own address; destination lane i receives element (i % 4) of source
lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.  The helpers (tr_frag<LD>, tr_frag_swz<R>
in ssd_lds.hpp, tr_h<R> in ssd_stream.hip) point source lane 4s + q of group g
at row k0 + 4g + s, elements r0 + 4q .. + 3."""
import numpy as np
import pytest


def swz(R, r):
    return r % 16 if R == 32 else (r // (16 // R)) % R


def off_plain(LD):
    return lambda r, e: r * LD + e


def off_swz(R):
    return lambda r, e: r * 8 * R + 8 * ((e >> 3) ^ swz(R, r)) + (e & 7)


def tr_load(mem, off, r0, k0):
    """Per-lane results of the transposing load and the byte addresses used."""
    out = np.zeros((64, 4), mem.dtype)
    addrs = []
    for g in range(4):
        src = {}
        for s in range(4):
            for q in range(4):
                a = off(k0 + 4 * g + s, r0 + 4 * q)
                addrs.append(2 * a)
                src[4 * s + q] = mem[a:a + 4]
        for i in range(16):
            for e in range(4):
                out[16 * g + i, e] = src[4 * e + i // 4][i % 4]
    return out, addrs


def direct(mem, off, r0, k0):
    out = np.zeros((64, 4), mem.dtype)
    for g in range(4):
        for i in range(16):
            for e in range(4):
                out[16 * g + i, e] = mem[off(k0 + 4 * g + e, r0 + i)]
    return out


def check(off, rows, cols, size, r0s, k0s):
    mem = np.arange(size, dtype=np.int64) * 7 + 3
    for r0 in r0s:
        for k0 in k0s:
            got, addrs = tr_load(mem, off, r0, k0)
            assert all(a % 8 == 0 for a in addrs), (r0, k0)
            assert all(0 <= a and a + 8 <= 2 * size for a in addrs), (r0, k0)
            assert k0 + 16 <= rows and r0 + 16 <= cols, (r0, k0)
            np.testing.assert_array_equal(got, direct(mem, off, r0, k0))


@pytest.mark.parametrize("P", [64, 128])
def test_backward_x_dy_and_state_tiles(P):
    """k_bwd_chunk: the dy (and x) tile of a 64-token chunk and the state
    halves, leading dimension P + 4; column tiles at K = 16 I, R = 16 pt."""
    LD, Q = P + 4, 64
    check(off_plain(LD), Q, P, Q * LD, [16 * pt for pt in range(P // 16)],
          [16 * i for i in range(Q // 16)])
    for NR in (16, 32, 64, 128):  # rows of a staged state part
        check(off_plain(LD), NR, P, NR * LD, [16 * pt for pt in range(P // 16)],
              [k for k in range(0, NR, 16)])


@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
def test_backward_b_c_tiles(N):
    """k_bwd_chunk: B and C of a 64-token chunk, leading dimension N + 4."""
    LD, Q = N + 4, 64
    check(off_plain(LD), Q, N, Q * LD, [16 * nt for nt in range(N // 16)],
          [16 * j for j in range(Q // 16)])


@pytest.mark.parametrize("Q", [64, 128, 256])
def test_fused_weighted_x_tile(Q):
    """k_fused: the weighted x tile, leading dimension P + 16 (P = 64)."""
    P = 64
    LD = P + 16
    check(off_plain(LD), Q, P, Q * LD, [16 * pt for pt in range(P // 16)],
          [k for k in range(0, Q, 16)])


@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
def test_stream_prep_b_slab(N):
    """k_stream_prep: a slab of up to 64 B rows, leading dimension N + 8."""
    LD, SR = N + 8, 64
    check(off_plain(LD), SR, N, SR * LD, [16 * nt for nt in range(N // 16)],
          [k for k in range(0, SR, 16)])


@pytest.mark.parametrize("R", [2, 4, 8, 16, 32])
def test_swizzled_tiles(R):
    """Swizzled unpadded tiles (x, B): 8 R elements per row, every 16-row
    block and 16-column tile."""
    rows, cols = 256, 8 * R
    check(off_swz(R), rows, cols, rows * cols, list(range(0, cols, 16)), list(range(0, rows, 16)))


def test_model_catches_misalignment():
    """The model rejects a leading dimension that is not a multiple of 4 (rows
    not 8-byte aligned) -- the compile-time check in tr_frag<LD>."""
    with pytest.raises(AssertionError):
        check(off_plain(66), 64, 64, 64 * 66, [0], [16])
