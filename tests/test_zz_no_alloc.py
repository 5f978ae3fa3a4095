"""The no-allocation entry point (ssd_fwd_noalloc): the library's own device
scratch buffer in place of a workspace argument.  Through the C ABI, two calls
in a row on different problems (the second smaller, so it runs on what the
first left in the buffer) give exactly what ssd_fwd gives with a workspace of
its own on the same inputs (same kernels, deterministic), and both match the
oracle; a problem that needs more scratch than the buffer holds is refused
with SSD_ERR_WORKSPACE before anything runs."""
import numpy as np
import pytest

import ssd_synth
from parity import TOL, compare, run_oracle, say, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _both(inp, algo):
    import ssd_scan_amd as ssd

    dev = to_device(inp)
    kw = dict(chunk_size=inp.chunk, dt_min=inp.dt_min, dt_max=inp.dt_max, algo=algo,
              scales_input=inp.scales_input, softplus=inp.softplus, return_final_states=True)
    y1, f1 = ssd.fwd(**dev, **kw)
    y2, f2 = ssd.fwd(**dev, **kw, library_scratch=True)
    torch.cuda.synchronize()
    return (y1.float().cpu().numpy(), f1.cpu().numpy()), (y2.float().cpu().numpy(), f2.cpu().numpy())


@pytest.mark.parametrize("algo", ["auto", "fused", "chunked"])
def test_noalloc_matches_workspace_entry_point(algo):
    first = ssd_synth.random_case(910, 2, 1000, 8, 64, 128, 2, chunk=256, dtype="bf16",
                                  with_init=True)
    second = ssd_synth.random_case(911, 1, 300, 4, 64, 64, 1, chunk=128, dtype="bf16",
                                   with_init=True)
    for k, inp in enumerate((first, second)):
        say(f"no-alloc call {k} algo={algo}")
        (y1, f1), (y2, f2) = _both(inp, algo)
        np.testing.assert_array_equal(y2, y1)
        np.testing.assert_array_equal(f2, f1)
        yr, fr = run_oracle(inp)
        ey, ef = compare(inp, y2, f2, yr, fr)
        assert ey < TOL["bf16"] and ef < TOL["bf16"], (ey, ef)


def test_noalloc_refuses_problems_beyond_the_buffer():
    import ssd_scan_amd as ssd

    # the chunked schedule's fp32 chunk states of this problem alone exceed 64 MiB
    x = torch.zeros(1, 65536, 32, 64, dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros(1, 65536, 32, dtype=torch.bfloat16, device="cuda")
    A = -torch.ones(32, device="cuda")
    B = torch.zeros(1, 65536, 1, 256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ssd.SsdError) as err:
        ssd.fwd(x, dt, A, B, B, algo="chunked", library_scratch=True)
    assert err.value.status == ssd.SSD_ERR_WORKSPACE
