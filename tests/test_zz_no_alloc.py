"""The allocation-free draft step (xpress_jacobi_step_noalloc) against the step with a caller
workspace (xpress_jacobi_step), through the C ABI.

Both run the same kernels, so the drafts and pass counts must be identical. Each case makes two
calls in a row on the library's static scratch, the second with fewer blocks and other values,
so anything the first call leaves in the scratch that the second would wrongly reuse shows up.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from jacobi_block_refiner_amd import synth, upload, xpress
from tests.gpu_helpers import Dev, log, strong

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    xpress.lib()
    torch.cuda.set_device(0)


def _both(d: Dev, *, K, C, flags):
    """(blk, passes) of the workspace step and of the allocation-free step on the same inputs."""
    wl = d.inp.wl
    outs = []
    for noalloc in (False, True):
        blk = upload.tokens(d.inp.blk)
        passes = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        if noalloc:
            xpress.jacobi_step_noalloc(d.w, d.h, d.base, d.anchor, d.am1, blk, K=K, C=C,
                                       flags=flags, passes_run=passes)
        else:
            ws = xpress.alloc_workspace(wl.N, wl.B, wl.r, wl.V, C, K)
            xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=K, C=C, flags=flags,
                               ws=ws, passes_run=passes)
        torch.cuda.synchronize()
        outs.append((blk.cpu().numpy(), int(passes.item())))
    return outs


@pytest.mark.parametrize("C", [0, 48])
@pytest.mark.parametrize("path", ["table", "project"])
def test_noalloc_step_equals_workspace_step_twice_in_a_row(C, path):
    flags = xpress.INIT_FROM_BASE | xpress.STOP_AT_FIXED_POINT
    for N, seed, K in ((6, 21, 16), (3, 22, 5)):  # second call: fewer blocks, other values
        inp = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=8), N=N, seed=seed))
        d = Dev(inp)
        if path == "project":
            d.w.w1p = None
        log(f"no-alloc step N={N} C={C} K={K} {path}")
        (blk_ws, p_ws), (blk_na, p_na) = _both(d, K=K, C=C, flags=flags)
        assert np.array_equal(blk_na, blk_ws)
        assert p_na == p_ws and 1 <= p_na <= K


def test_noalloc_step_at_full_size_then_fewer_blocks():
    """The 32-block full-vocabulary workload (V = 151936, K = 15, the benchmark's flags), then 8
    blocks of another draw, fixed K."""
    for N, seed, flags in ((32, 0, xpress.INIT_FROM_BASE),
                           (8, 3, xpress.INIT_FROM_BASE | xpress.STOP_AT_FIXED_POINT)):
        log(f"no-alloc full-size step N={N} seed={seed}")
        d = Dev(synth.make_inputs(3, seed=seed, N=N))
        (blk_ws, p_ws), (blk_na, p_na) = _both(d, K=15, C=0, flags=flags)
        assert np.array_equal(blk_na, blk_ws)
        assert p_na == p_ws
        del d
        torch.cuda.empty_cache()


def test_noalloc_step_rejects_more_than_its_scratch():
    """A step that needs more than the static scratch (512 blocks of the full-vocabulary shape
    need ~87 MiB of its 64 MiB) is refused on the host with XPRESS_ERR_WORKSPACE; nothing runs.
    The inputs cover all 512 blocks all the same, so nothing would be read out of bounds even if
    the step ran."""
    inp = synth.make_inputs(replace(synth.WORKLOADS[1], B=16, r=256, V=151936, M=512), N=1)
    d = Dev(inp)
    dims = d.w.dims
    N, B, V = 512, dims["B"], dims["V"]
    assert xpress.workspace_size(N, B, dims["r"], V, 0, 15) > 80 << 20
    h = torch.zeros(N, B, dims["H"], dtype=torch.bfloat16, device="cuda")
    base = torch.zeros(N * (B - 1), V, dtype=torch.bfloat16, device="cuda")
    anchor = torch.zeros(N, dtype=torch.int64, device="cuda")
    blk = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    with pytest.raises(xpress.XpressError) as e:
        xpress.jacobi_step_noalloc(d.w, h, base, anchor, anchor, blk, K=15, C=0)
    assert e.value.status == xpress.ERR_WORKSPACE
    assert "static scratch" in str(e.value)
    assert int(blk.abs().sum().item()) == 0
    del h, base
    torch.cuda.empty_cache()
