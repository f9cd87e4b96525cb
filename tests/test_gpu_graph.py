"""A draft step recorded as a HIP graph (xpress_jacobi_step_graph) and replayed.

Every replay must equal the eager step on the same inputs, bit for bit (same kernels, same
order). The replays are interleaved with eager work and synchronizations, the inputs the graph
reads are rewritten between replays (the graph must pick up the new values), and blk is reset
eagerly before each replay so a replay that did nothing would be caught.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from jacobi_block_refiner_amd import synth, upload, xpress
from tests.gpu_helpers import Dev, log, strong

pytestmark = pytest.mark.gpu


def _eager(d, base, blk0, K, flags, C=0):
    blk = blk0.clone()
    passes = torch.zeros(1, dtype=torch.int32, device="cuda")
    xpress.jacobi_step(d.w, d.h, base, d.anchor, d.am1, blk, K=K, C=C, flags=flags,
                       ws=d.ws(C=C, K=K), passes_run=passes)
    torch.cuda.synchronize()
    return blk.cpu().numpy(), int(passes.item())


@pytest.mark.parametrize("flags", [xpress.INIT_FROM_BASE | xpress.STOP_AT_FIXED_POINT,
                                   xpress.INIT_FROM_BASE, 0])
@pytest.mark.parametrize("C", [0, 64])
def test_graph_replays_equal_eager_steps(flags, C):
    inp = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=8), N=6, seed=5))
    N, B = inp.blk.shape
    K = B
    d = Dev(inp)
    blk0 = upload.tokens(inp.blk)
    # a second set of base logits, written into the graph's own base buffer between replays
    inp2 = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=8), N=6, seed=6))
    base2 = upload.base_logits(inp2.base)

    want1 = _eager(d, d.base, blk0, K, flags, C)
    want2 = _eager(d, base2, blk0, K, flags, C)

    base = d.base.clone()  # the buffer the graph records
    blk = blk0.clone()
    passes = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = d.ws(C=C, K=K)
    g = xpress.StepGraph(d.w, d.h, base, d.anchor, d.am1, blk, K=K, C=C, flags=flags, ws=ws,
                         passes_run=passes)
    torch.cuda.synchronize()
    assert np.array_equal(blk.cpu().numpy(), blk0.cpu().numpy())  # recording ran nothing
    try:
        for rep, (src, want) in enumerate([(d.base, want1), (base2, want2), (d.base, want1),
                                           (d.base, want1)]):
            base.copy_(src)                 # eager work between replays
            blk.copy_(blk0)
            passes.zero_()
            torch.cuda.synchronize()
            g.launch()
            torch.cuda.synchronize()
            got = blk.cpu().numpy(), int(passes.item())
            log(f"graph C={C} flags={flags} replay {rep}: passes {got[1]} (eager {want[1]})")
            assert np.array_equal(got[0], want[0])
            assert got[1] == want[1]
    finally:
        g.close()


def test_graph_argument_errors_and_destroy():
    inp = synth.make_inputs(1).rounded_bf16()
    d = Dev(inp)
    blk = upload.tokens(inp.blk)
    with pytest.raises(xpress.XpressError):
        xpress.StepGraph(d.w, d.h, d.base, d.anchor, d.am1, blk, K=2, flags=0x80, ws=d.ws())
    with pytest.raises(xpress.XpressError):  # workspace too small
        xpress.StepGraph(d.w, d.h, d.base, d.anchor, d.am1, blk, K=2,
                         ws=torch.empty(256, dtype=torch.uint8, device="cuda"))
    g = xpress.StepGraph(d.w, d.h, d.base, d.anchor, d.am1, blk, K=2, ws=d.ws())
    g.close()
    g.close()  # idempotent
    with pytest.raises(RuntimeError):
        g.launch()
    assert xpress.lib().xpress_graph_destroy(None) == xpress.OK


def test_binding_refuses_inputs_that_do_not_cover_n_blocks():
    """The C ABI takes bare pointers and N (from blk's first dimension): the binding refuses, on
    the host and before any call, inputs that cover fewer blocks than blk asks for."""
    inp = synth.make_inputs(1).rounded_bf16()
    d = Dev(inp)
    N, B = inp.blk.shape
    more = torch.zeros(N + 1, B, dtype=torch.int64, device="cuda")
    for step in (lambda blk: xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=2,
                                                ws=d.ws()),
                 lambda blk: xpress.jacobi_step_noalloc(d.w, d.h, d.base, d.anchor, d.am1, blk,
                                                        K=2),
                 lambda blk: xpress.StepGraph(d.w, d.h, d.base, d.anchor, d.am1, blk, K=2,
                                              ws=d.ws()),
                 lambda blk: xpress.initial_block(d.base, d.anchor, blk)):
        with pytest.raises(ValueError):
            step(more)
    torch.cuda.synchronize()
    assert int(more.abs().sum().item()) == 0
