"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The GPU runs every block; the oracle recomputes sampled blocks (blocks are independent: no term
of the pass mixes two blocks), and properties that hold at any size are checked on every block:
  * one pass from the drawn block: tokens agree with the oracle on sampled blocks (near-tie rule),
    latents within the row-relative tolerance;
  * a K = B-1 step reaches a fixed point (one more pass changes nothing), is deterministic, and
    agrees end to end with the oracle on sampled blocks (near-tie cascade rule);
  * top-C: candidate sets, gathered base logits and readout rows are bit-exact on sampled rows and
    every drafted token is a candidate of its row.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from jacobi_block_refiner_amd import synth, upload, xpress
from oracle import oracle as O
from tests.gpu_helpers import (LAT_RTOL, Dev, compare_tokens, draft_rows, end_to_end_ok,
                               lat_rel_err, lat_to_f64, log, oracle_mixer)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

_cache = {}


def _dev(wl_id):
    if wl_id not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        log(f"workload {wl_id}: drawing inputs")
        inp = synth.make_inputs(wl_id)
        log(f"workload {wl_id}: uploading")
        _cache[wl_id] = Dev(inp)
    return _cache[wl_id]


def _subset(inp, blocks):
    B = inp.wl.B
    rows = (np.asarray(blocks)[:, None] * (B - 1) + np.arange(B - 1)[None, :]).reshape(-1)
    return replace(inp, wl=replace(inp.wl, N=len(blocks)), h=inp.h[blocks],
                   base=inp.base[rows], blk=inp.blk[blocks], am1=inp.am1[blocks]), rows


def _sample_blocks(N, k):
    return sorted(set(np.linspace(0, N - 1, num=min(k, N)).astype(int).tolist()))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    xpress.lib()
    yield
    _cache.clear()


# 256 blocks: 8 sampled blocks, one in each 512-row chunk of the readout
@pytest.mark.parametrize("wl_id,n_sample", [(2, 1), (3, 3), (5, 8)])
def test_one_pass_full_vocab(wl_id, n_sample):
    d = _dev(wl_id)
    inp = d.inp
    log(f"workload {wl_id}: one pass on the GPU")
    xh = d.xh()
    got, lat = d.one_pass(inp.blk, xh)
    assert np.array_equal(got[:, 0], inp.blk[:, 0])
    blocks = _sample_blocks(inp.wl.N, n_sample)
    sub, rows = _subset(inp, blocks)
    log(f"workload {wl_id}: oracle on blocks {blocks}")
    L = oracle_mixer(inp)
    xh_o = O.hidden_cache(sub.h, sub.down_h, sub.down_g, sub.in_proj)
    lat_o = O.latent(sub, L, xh_o, sub.blk, sub.am1)
    err = lat_rel_err(lat_to_f64(lat)[blocks], lat_o)
    best, gap, _ = O.readout_argmax(lat_o.reshape(-1, inp.wl.r), sub.w2, sub.base)
    bad, exempt = compare_tokens(draft_rows(got[blocks]), best, gap)
    log(f"workload {wl_id}: latent error {err:.2e}; token mismatches {bad}, near ties {exempt}")
    assert err < LAT_RTOL
    assert bad == 0


@pytest.mark.parametrize("wl_id,n_sample", [(2, 1), (3, 2), (5, 3)])
def test_step_reaches_fixed_point_and_matches_oracle(wl_id, n_sample):
    d = _dev(wl_id)
    inp, wl = d.inp, d.inp.wl
    K = wl.B - 1
    ws = d.ws(K=K + 1)
    outs = []
    for rep in range(2):
        log(f"workload {wl_id}: step K={K} run {rep}")
        blk = torch.zeros(wl.N, wl.B, dtype=torch.int64, device="cuda")
        xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=K, flags=xpress.INIT_FROM_BASE,
                           ws=ws)
        torch.cuda.synchronize()
        outs.append(blk)
    assert torch.equal(outs[0], outs[1])
    blk = outs[0]
    changed = torch.zeros(1, dtype=torch.int32, device="cuda")
    lat = torch.empty(wl.N, wl.B - 1, wl.r, dtype=torch.bfloat16, device="cuda")
    xh = d.xh()
    after = blk.clone()
    xpress.latent_pass(d.w, after, d.am1, xh, lat, ws)
    xpress.readout_argmax(d.w, lat, d.base, after, ws, changed)
    torch.cuda.synchronize()
    assert int(changed.item()) == 0 and torch.equal(after, blk)
    got = blk.cpu().numpy()
    blocks = _sample_blocks(wl.N, n_sample)
    sub, _ = _subset(inp, blocks)
    log(f"workload {wl_id}: oracle Jacobi on blocks {blocks}")
    L = oracle_mixer(inp)
    xh_o = O.hidden_cache(sub.h, sub.down_h, sub.down_g, sub.in_proj)
    start = O.initial_block(sub.base, sub.blk[:, 0], len(blocks), wl.B)
    want, _, _, hg = O.jacobi(sub, L, xh_o, start, K=K, stop_at_fixed_point=False, history=True)
    bad, exempt = end_to_end_ok(got[blocks], want, hg)
    log(f"workload {wl_id}: end-to-end disallowed mismatches {bad}, near-tie row-passes {exempt}")
    assert bad == 0


def test_topc_full_size():
    d = _dev(4)
    inp, wl = d.inp, d.inp.wl
    C = wl.C
    rows = wl.rows
    cand = torch.empty(rows, C, dtype=torch.int64, device="cuda")
    base_c = torch.empty(rows, C, dtype=torch.bfloat16, device="cuda")
    w2c = torch.empty(rows, C, wl.r, dtype=torch.bfloat16, device="cuda")
    log("workload 4: top-C prepare")
    xpress.topc_prepare(d.w, d.base, wl.N, C, cand, base_c, w2c)
    torch.cuda.synchronize()
    sample_rows = np.arange(0, rows, 37)
    want = O.topc_select(inp.base[sample_rows], C)
    got = cand.cpu().numpy()
    assert np.array_equal(got[sample_rows], want)
    assert np.all(np.diff(got, axis=1) > 0)  # ascending ids, no duplicates, on every row
    assert np.array_equal(base_c.float().cpu().numpy()[sample_rows],
                          np.take_along_axis(inp.base[sample_rows], want, axis=1))
    w2c_s = w2c[torch.from_numpy(sample_rows).cuda()].float().cpu().numpy()
    assert np.array_equal(w2c_s, inp.w2[want])
    # every row: the candidates hold the C largest keys (no id outside has a larger value than
    # an id inside)
    base_t = d.base.float()
    inside_min = torch.gather(base_t, 1, cand).min(dim=1).values
    mask = torch.ones_like(base_t, dtype=torch.bool).scatter_(1, cand, False)
    outside_max = torch.where(mask, base_t, torch.full_like(base_t, -float("inf"))).max(dim=1).values
    assert bool((outside_max <= inside_min).all())

    log("workload 4: one top-C pass")
    xh = d.xh()
    got_blk, lat = d.one_pass(inp.blk, xh, cand=cand, base_c=base_c, w2c=w2c)
    blocks = _sample_blocks(wl.N, 3)
    sub, sub_rows = _subset(inp, blocks)
    L = oracle_mixer(inp)
    xh_o = O.hidden_cache(sub.h, sub.down_h, sub.down_g, sub.in_proj)
    lat_o = O.latent(sub, L, xh_o, sub.blk, sub.am1)
    cand_o = O.topc_select(sub.base, C)
    best, gap, _ = O.readout_argmax(lat_o.reshape(-1, wl.r), sub.w2, sub.base, cand=cand_o)
    bad, exempt = compare_tokens(draft_rows(got_blk[blocks]), best, gap)
    log(f"workload 4: latent error {lat_rel_err(lat_to_f64(lat)[blocks], lat_o):.2e}; "
        f"token mismatches {bad}, near ties {exempt}")
    assert bad == 0
    cc = cand.cpu().numpy()
    dr = draft_rows(got_blk)
    assert all(dr[p] in cc[p] for p in range(rows))

    log("workload 4: the selection with chunk maxima (the form a step runs)")
    cand2 = torch.empty_like(cand)
    base_c2 = torch.empty_like(base_c)
    ws = d.ws(C=C, K=wl.B)
    xpress.topc_prepare(d.w, d.base, wl.N, C, cand2, base_c2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(cand2, cand) and torch.equal(base_c2, base_c)  # every row
    rows_s2 = np.arange(5, rows, 41)
    assert np.array_equal(cand2.cpu().numpy()[rows_s2], O.topc_select(inp.base[rows_s2], C))

    log("workload 4: step with top-C, K=B-1 as the benchmark runs it, then one more pass")
    K = wl.B - 1
    blk = torch.zeros(wl.N, wl.B, dtype=torch.int64, device="cuda")
    xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=K, C=C,
                       flags=xpress.INIT_FROM_BASE, ws=ws)
    after = blk.clone()
    changed = torch.zeros(1, dtype=torch.int32, device="cuda")
    lat2 = torch.empty(wl.N, wl.B - 1, wl.r, dtype=torch.bfloat16, device="cuda")
    xpress.latent_pass(d.w, after, d.am1, xh, lat2, ws)
    xpress.readout_argmax_topc(lat2, w2c, base_c, cand, after, changed)
    torch.cuda.synchronize()
    assert int(changed.item()) == 0 and torch.equal(after, blk)
    got = blk.cpu().numpy()
    assert all(tok in cc[p] for p, tok in enumerate(draft_rows(got)))
    blocks = _sample_blocks(wl.N, 3)
    sub, _ = _subset(inp, blocks)
    log(f"workload 4: oracle top-C Jacobi on blocks {blocks}")
    xh_o = O.hidden_cache(sub.h, sub.down_h, sub.down_g, sub.in_proj)
    cand_o = O.topc_select(sub.base, C)
    start = O.initial_block(sub.base, sub.blk[:, 0], len(blocks), wl.B)
    want, _, _, hg = O.jacobi(sub, L, xh_o, start, K=K, stop_at_fixed_point=False, cand=cand_o,
                              history=True)
    bad, exempt = end_to_end_ok(got[blocks], want, hg)
    log(f"workload 4: end-to-end disallowed mismatches {bad}, near-tie row-passes {exempt}")
    assert bad == 0
