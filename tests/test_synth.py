"""The seeded input generator: bf16 rounding and the workload recipes."""
import numpy as np
import torch

from jacobi_block_refiner_amd import synth


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, -0.0,
                                  3.0e38, 1e-40], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), want)
    assert np.array_equal(synth.bits_to_f32(want), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workloads_are_deterministic_and_shaped():
    a = synth.make_inputs(1)
    b = synth.make_inputs(1)
    for k in synth.Inputs.FLOAT_FIELDS + ("blk", "am1"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    wl = a.wl
    assert a.base.shape == (wl.N * (wl.B - 1), wl.V) and a.w2.shape == (wl.V, wl.r)
    assert a.blk.min() >= 0 and a.blk.max() < wl.V and a.blk.dtype == np.int64
    r = a.rounded_bf16()
    assert np.array_equal(r.w1, synth.bf16_round(a.w1))


def test_bf16_workload_values_are_bf16_and_boosted():
    wl = synth.WORKLOADS[2]
    inp = synth.make_inputs(2)
    for k in ("w1", "w2", "base", "raw_L", "h"):
        v = getattr(inp, k)
        assert np.array_equal(v, synth.bf16_round(v))
    ids = inp.meta["boost_ids"]
    assert ids.shape == (wl.rows,)
    # the boosted logits sit far in the upper tail of N(0, 2)
    assert np.mean(inp.base[np.arange(wl.rows), ids]) > 4.0
