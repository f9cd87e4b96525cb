"""GPU parity of each kernel of the XPress pass against the CPU oracle, on small seeded inputs
that span several tiles and a ragged tail. Every call goes through the C ABI."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from jacobi_block_refiner_amd import synth, upload, xpress
from oracle import oracle as O
from tests.gpu_helpers import (LAT_RTOL, NEAR_TIE, Dev, compare_tokens, draft_rows, end_to_end_ok,
                               lat_pack_fragments, lat_rel_err, lat_to_f64,
                               lat_unpack_fragments, log, oracle_mixer, strong)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    xpress.lib()
    torch.cuda.set_device(0)


def _dyadic(rng, shape, lo, hi, den):
    return (rng.integers(lo, hi + 1, size=shape) / den).astype(np.float32)


def _readout_case(seed, N, B, r, V, *, zero_head=False):
    """Dyadic lat / w2 / base (exact in bf16 and in every fp32 partial sum) with planted ties."""
    rng = np.random.default_rng(seed)
    rows = N * (B - 1)
    lat = _dyadic(rng, (rows, r), -4, 4, 16)
    w2 = np.zeros((V, r), np.float32) if zero_head else _dyadic(rng, (V, r), -4, 4, 16)
    base = _dyadic(rng, (rows, V), -8, 8, 4)
    for p in range(0, rows, 3):  # exact top ties between a high and a low id (distinct pairs)
        hi, lo = V - 1 - p, p
        w2[lo] = w2[hi]
        base[p, hi] = base[p, lo] = 31.75
    return lat, w2, base


def _weights_with(w2_np, r, B, V, device="cuda"):
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16, device=device)
    return xpress.Weights(w1=z(V, r), down_h=z(r, 64), down_g=z(r, 64), in_proj=z(r, 3 * r),
                          mix_L=z(B, B, r), w_gate=z(64, r), w_up=z(64, r), w_down=z(r, 64),
                          w2=upload.bf16_tensor(w2_np, device))


# ----------------------------------------------------------------------------------------------

def test_fold_mixer_bit_exact():
    rng = np.random.default_rng(0)
    for r, B in ((64, 4), (256, 16)):
        raw = synth.bf16_round(rng.standard_normal((r, B, B)).astype(np.float32) * 0.05)
        got = xpress.fold_mixer(upload.bf16_tensor(raw)).float().cpu().numpy()
        assert got.shape == (B, B, r)  # stored channel innermost
        inp = replace(synth.make_inputs(1), raw_L=raw)
        assert np.array_equal(got.transpose(2, 0, 1).astype(np.float64), oracle_mixer(inp))


@pytest.mark.parametrize("V", [5003, 8192])
def test_initial_block_exact(V):
    rng = np.random.default_rng(1)
    N, B = 5, 16
    rows = N * (B - 1)
    base = synth.bf16_round(rng.standard_normal((rows, V)).astype(np.float32) * 2)
    top = base.argmax(1)
    for p in range(0, rows, 2):  # duplicated maxima below and above the first one
        base[p, (top[p] + 1 + p) % V] = base[p, top[p]]
    base[3, :] = 0.0
    base[3, 17] = -0.0  # -0 ties +0; id 0 must win
    anchor = rng.integers(0, V, N)
    blk = torch.full((N, B), -1, dtype=torch.int64, device="cuda")
    xpress.initial_block(upload.base_logits(base), upload.tokens(anchor), blk)
    torch.cuda.synchronize()
    want = O.initial_block(base, anchor, N, B)
    assert np.array_equal(blk.cpu().numpy(), want)


# N = 1 and 2 (15 and 30 rows) take the one-tile shape (the long vocabularies give ranges of
# several steps, so the ring wraps); N = 20 and 35 (300 and 525 rows)
# take the wide row-chunk shape; 525 rows span two row chunks
@pytest.mark.parametrize("r,V,N", [(64, 5003, 3), (256, 5003, 5), (256, 8192, 3), (128, 700, 2),
                                   (256, 151936, 1), (128, 60001, 2), (64, 40000, 1),
                                   (256, 5003, 20), (256, 8192, 35), (128, 3001, 35)])
@pytest.mark.parametrize("layout", ["rows", "fragments"])
def test_readout_argmax_dyadic_exact(r, V, N, layout):
    """Every fp32 partial sum is exact, so the GPU must match the oracle on every row, ties
    included (lowest id), with no near-tie exemption. lat is given row-major or in the fragment
    order a step keeps it in (a permutation of the same values)."""
    B = 16
    lat, w2, base = _readout_case(2, N, B, r, V)
    w = _weights_with(w2, r, B, V)
    rng = np.random.default_rng(3)
    blk0 = rng.integers(0, V, (N, B))
    blk = upload.tokens(blk0)
    changed = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = xpress.alloc_workspace(N, B, r, V, 0, 1)
    log(f"readout dyadic r={r} V={V} N={N} lat {layout}")
    if layout == "rows":
        lat_d, lay = upload.bf16_tensor(lat), xpress.LAT_ROWS
    else:
        lat_d, lay = upload.bf16_tensor(lat_pack_fragments(lat)), xpress.LAT_FRAGMENTS
    xpress.readout_argmax(w, lat_d, upload.base_logits(base), blk, ws, changed, layout=lay)
    torch.cuda.synchronize()
    best, gap, _ = O.readout_argmax(lat, w2, base)
    got = blk.cpu().numpy()
    assert np.array_equal(got[:, 0], blk0[:, 0])  # the anchor slot is never written
    assert np.array_equal(draft_rows(got), best)
    assert (gap == 0).sum() >= len(range(0, N * (B - 1), 3))
    assert int(changed.item()) == int(not np.array_equal(draft_rows(blk0), best))


# 45 rows: one row chunk, 256 ranges; 600 and 1800 rows: two and four chunks of 512 rows, so
# 128 and 64 longer ranges; V = 3001 at 600 rows: 94 ranges of one or two steps (not a multiple
# of 8, so the plain workgroup order rather than the per-XCD one)
@pytest.mark.parametrize("r,V,N", [(128, 8192, 3), (128, 8195, 40), (64, 20000, 120),
                                   (128, 3001, 40)])
def test_readout_partials_per_range_and_reduce(r, V, N):
    """The two-stage readout through the C ABI: each (range, row) partial is the exact maximum
    and lowest id over range t = steps [S*t // ntiles, S*(t+1) // ntiles) of the S = ceil(V/32)
    32-id steps (dyadic values, so every fp32 sum is exact), and their reduce gives the one-call
    readout's block."""
    B = 16
    rows = N * (B - 1)
    lat, w2, base = _readout_case(6, N, B, r, V)
    w = _weights_with(w2, r, B, V)
    ntiles = xpress.readout_tiles(V, rows)
    S = (V + 31) // 32
    want_nt = min(S, 256 if rows <= 512 else max(8, (256 // -(-rows // 512)) & ~7))
    assert ntiles == want_nt
    part = torch.full((ntiles, rows, 2), -1, dtype=torch.int32, device="cuda")
    lat_d, base_d = upload.bf16_tensor(lat), upload.base_logits(base)
    log(f"readout partials r={r} V={V} N={N} ntiles={ntiles}")
    xpress.readout_partials(w, lat_d, base_d, part)
    blk_two = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    xpress.argmax_reduce(part, blk_two)
    blk_one = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    xpress.readout_argmax(w, lat_d, base_d, blk_one, xpress.alloc_workspace(N, B, r, V, 0, 1))
    torch.cuda.synchronize()
    got = part.cpu().numpy()
    for t in range(ntiles):
        a, b = 32 * (S * t // ntiles), min(V, 32 * (S * (t + 1) // ntiles))
        best, _, val = O.readout_argmax(lat, w2[a:b], np.ascontiguousarray(base[:, a:b]))
        assert np.array_equal(got[t, :, 1], best + a), t
        assert np.array_equal(got[t, :, 0].view(np.float32), val.astype(np.float32)), t
    full, _, _ = O.readout_argmax(lat, w2, base)
    assert np.array_equal(draft_rows(blk_two.cpu().numpy()), full)
    assert torch.equal(blk_two, blk_one)


# A base row stride of 2^23 elements: a 512-row chunk (32 blocks) spans 8 GB of base and a
# 256-row chunk (17 blocks) 4.3 GB, beyond what a 32-bit byte offset from one pointer reaches; a
# single request's 32-row chunk stays below it
@pytest.mark.parametrize("N", [1, 17, 32])
def test_readout_and_starting_block_with_a_large_base_stride(N):
    B, r, V, LD = 16, 256, 5003, 1 << 23
    lat, w2, base = _readout_case(11, N, B, r, V)
    w = _weights_with(w2, r, B, V)
    dense = upload.base_logits(base)
    log(f"readout with base_ld = 2^23, N={N}")
    big = torch.empty((dense.shape[0], LD), dtype=torch.bfloat16, device="cuda")
    big[:, :8 * -(-V // 8)].zero_()  # the row padding up to a multiple of 8 ids
    view = big[:, :V]
    view.copy_(dense)
    assert view.stride(0) == LD
    ws = xpress.alloc_workspace(N, B, r, V, 0, 1)
    blk_big = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    xpress.readout_argmax(w, upload.bf16_tensor(lat), view, blk_big, ws)
    anchor = upload.tokens(np.arange(N))
    start = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    xpress.initial_block(view, anchor, start)
    torch.cuda.synchronize()
    best, _, _ = O.readout_argmax(lat, w2, base)
    assert np.array_equal(draft_rows(blk_big.cpu().numpy()), best)
    want = O.initial_block(base, np.arange(N), N, B)
    assert np.array_equal(start.cpu().numpy(), want)
    del big, view
    torch.cuda.empty_cache()


@pytest.mark.parametrize("V", [1, 7, 31, 33])
def test_readout_argmax_small_vocabulary(V):
    """A vocabulary of fewer ids than one 32-id step (or just past it): the single partial step's
    ids past V must never win; dyadic values, so the argmax is exact (ties included)."""
    N, B, r = 2, 16, 64
    rows = N * (B - 1)
    rng = np.random.default_rng(11 + V)
    lat = _dyadic(rng, (rows, r), -4, 4, 16)
    w2 = _dyadic(rng, (V, r), -4, 4, 16)
    base = _dyadic(rng, (rows, V), -8, 8, 4)
    blk = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    log(f"readout small vocabulary V={V}")
    xpress.readout_argmax(_weights_with(w2, r, B, V), upload.bf16_tensor(lat),
                          upload.base_logits(base), blk, xpress.alloc_workspace(N, B, r, V, 0, 1))
    torch.cuda.synchronize()
    best, _, _ = O.readout_argmax(lat, w2, base)
    assert np.array_equal(draft_rows(blk.cpu().numpy()), best)


def test_readout_zero_head_is_argmax_of_base():
    N, B, r, V = 4, 16, 256, 4099
    lat, w2, base = _readout_case(4, N, B, r, V, zero_head=True)
    lat = lat * 1000
    w = _weights_with(w2, r, B, V)
    blk = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    xpress.readout_argmax(w, upload.bf16_tensor(lat), upload.base_logits(base), blk,
                          xpress.alloc_workspace(N, B, r, V, 0, 1))
    torch.cuda.synchronize()
    assert np.array_equal(draft_rows(blk.cpu().numpy()), np.argmax(base, axis=1))


def test_readout_start_and_selection_at_the_largest_vocabulary():
    """V = 2^31/r - 1 at r = 256 (8,388,607 ids, the most the library takes; ids up to 2^23 and
    w2 offsets up to 2^31 bytes). A zero head leaves the readout the argmax of base, so the draft
    is np.argmax (lowest id on ties, one planted at both ends of a row); the starting block is the
    same argmax; a top-64 selection (the exact path: rows past 524,288 ids) matches the oracle."""
    N, B, r = 1, 16, 256
    V = (1 << 31) // r - 1
    rows = N * (B - 1)
    rng = np.random.default_rng(12)
    base = synth.bf16_round(rng.standard_normal((rows, V), dtype=np.float32) * 3)
    base[3, V - 1] = base[3, 17] = 40.0
    z = lambda *shape: torch.zeros(*shape, dtype=torch.bfloat16, device="cuda")
    w = xpress.Weights(w1=z(V, r), down_h=z(r, 64), down_g=z(r, 64), in_proj=z(r, 3 * r),
                       mix_L=z(B, B, r), w_gate=z(64, r), w_up=z(64, r), w_down=z(r, 64),
                       w2=z(V, r))
    base_d = upload.base_logits(base)
    log(f"readout, starting block and top-64 at V={V}")
    blk = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    xpress.readout_argmax(w, z(rows, r), base_d, blk, xpress.alloc_workspace(N, B, r, V, 0, 1))
    start = torch.zeros(N, B, dtype=torch.int64, device="cuda")
    xpress.initial_block(base_d, upload.tokens(np.array([5])), start)
    cand = torch.empty(rows, 64, dtype=torch.int64, device="cuda")
    base_c = torch.empty(rows, 64, dtype=torch.bfloat16, device="cuda")
    xpress.topc_prepare(w, base_d, N, 64, cand, base_c)
    torch.cuda.synchronize()
    want = np.argmax(base, axis=1)
    assert want[3] == 17
    assert np.array_equal(draft_rows(blk.cpu().numpy()), want)
    assert np.array_equal(start.cpu().numpy()[0], np.concatenate([[5], want]))
    assert np.array_equal(cand.cpu().numpy(), O.topc_select(base, 64))
    del w, base_d
    torch.cuda.empty_cache()


def test_readout_changed_flag_stays_clear_at_a_fixed_point():
    N, B, r, V = 2, 16, 64, 3000
    lat, w2, base = _readout_case(5, N, B, r, V)
    best, _, _ = O.readout_argmax(lat, w2, base)
    blk0 = np.zeros((N, B), np.int64)
    blk0[:, 1:] = best.reshape(N, B - 1)
    blk = upload.tokens(blk0)
    changed = torch.zeros(1, dtype=torch.int32, device="cuda")
    xpress.readout_argmax(_weights_with(w2, r, B, V), upload.bf16_tensor(lat),
                          upload.base_logits(base), blk, xpress.alloc_workspace(N, B, r, V, 0, 1),
                          changed)
    torch.cuda.synchronize()
    assert int(changed.item()) == 0 and np.array_equal(blk.cpu().numpy(), blk0)


# the last two run the GEMM's deep path (a slice's chunks loaded 8 at a time): 16 chunks per
# slice, and 20 (16 + a remainder of 4) with a ragged last row tile (528 slot rows)
# H = 16384: the largest hidden size the library takes (256 k chunks over the split-K slices);
# N = 256: one split, a projection workgroup of 64 channels per block
@pytest.mark.parametrize("H,r,N,B", [(256, 64, 3, 4), (4096, 256, 3, 16), (320, 128, 2, 7),
                                     (4096, 256, 32, 16), (5120, 256, 33, 16), (16384, 256, 3, 16),
                                     (1024, 256, 256, 16)])
def test_hidden_cache_parity(H, r, N, B):
    base_wl = synth.WORKLOADS[1] if r == 64 else synth.WORKLOADS[3]
    wl = replace(base_wl, N=N, B=B, H=H, r=r, V=512, M=128)
    inp = synth.make_inputs(wl).rounded_bf16()
    d = Dev(inp)
    got = d.xh().cpu().numpy().astype(np.float64)
    want = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    err = lat_rel_err(got, want)
    log(f"hidden cache H={H} r={r}: row-relative error {err:.2e}")
    assert err < 1e-4


def _latent_case(wl_id, N, seed=0, **over):
    wl = replace(synth.WORKLOADS[wl_id], N=N, **over)
    inp = synth.make_inputs(wl, seed=seed).rounded_bf16()
    rng = np.random.default_rng(seed + 100)
    xh = (rng.standard_normal((N, wl.B, wl.r)) * 0.5).astype(np.float32)
    return inp, xh


def _dev(inp, path):
    """Device inputs; path "table": the latent gathers the projected embedding table (two
    launches); "project": it projects the gathered w1 rows itself (three launches)."""
    d = Dev(inp)
    if path == "project":
        d.w.w1p = None
    else:
        assert d.w.w1p is not None
    return d


@pytest.mark.parametrize("r,V", [(64, 1000), (128, 4096), (256, 8195)])
def test_fold_embedding_matches_oracle_projection(r, V):
    """w1p[v] = P_e . w1[v]: the oracle's latent with an identity mixer and a zero hidden cache
    returns exactly that projection as its mixer output u, for the ids the slots read."""
    wl = replace(synth.WORKLOADS[1], N=4, B=16, r=r, V=V, M=64)
    inp = synth.make_inputs(wl, seed=5).rounded_bf16()
    d = Dev(inp)
    got_all = d.w.w1p.cpu().numpy().astype(np.float64)
    assert got_all.shape == (V, r)
    rng = np.random.default_rng(7)
    ids = np.concatenate([[0, V - 1, V // 2], rng.integers(0, V, size=4 * 16 - 3)])
    blk = ids[: 4 * 16].reshape(4, 16)
    am1 = rng.integers(0, V, size=4)
    L = np.broadcast_to(np.eye(16), (r, 16, 16)).copy()
    _, u = O.latent(replace(inp, am1=am1), L, np.zeros((4, 16, r)), blk, am1, return_u=True)
    prev = np.concatenate([am1[:, None], blk[:, :-1]], axis=1)  # ids read by the 16 slots
    got = got_all[prev.reshape(-1)]
    err = lat_rel_err(got, u.reshape(-1, r))
    log(f"fold embedding r={r} V={V}: row-relative error {err:.2e}")
    assert err < 1e-5


@pytest.mark.parametrize("path", ["table", "project"])
@pytest.mark.parametrize("wl_id,N,over", [(1, 3, {}), (3, 3, {"V": 4096}),
                                         (1, 2, {"B": 7, "M": 256, "r": 128}),
                                         (3, 2, {"V": 2048, "M": 1024}),
                                         (1, 37, {"B": 16, "r": 256, "M": 512, "V": 3000}),
                                         (1, 5, {"B": 2, "r": 64, "M": 64, "V": 700}),
                                         # at M = 512 the table path takes up to 56 blocks (448
                                         # share workgroups, two per CU); from 57 on the
                                         # three-kernel path runs, table or not
                                         (1, 32, {"B": 16, "r": 256, "M": 512, "V": 3000}),
                                         (1, 33, {"B": 16, "r": 256, "M": 512, "V": 3000}),
                                         (1, 56, {"B": 16, "r": 256, "M": 512, "V": 3000}),
                                         (1, 57, {"B": 16, "r": 256, "M": 512, "V": 3000}),
                                         (1, 96, {"B": 16, "r": 256, "M": 512, "V": 3000}),
                                         (1, 130, {"B": 16, "r": 256, "M": 512, "V": 3000}),
                                         # the slice width follows N * M/32 <= 256 (32 units) and the
                                         # path N * M/64 <= 448: M = 1024 at 12 and 28 blocks takes
                                         # 64-unit slices on the table path, M = 256 at 20 and 40
                                         # blocks 32- and 64-unit ones, at 113 blocks the
                                         # three-kernel path
                                         (3, 12, {"V": 2048, "M": 1024}),
                                         (3, 28, {"V": 2048, "M": 1024}),
                                         (1, 20, {"B": 16, "r": 256, "M": 256, "V": 3000}),
                                         (1, 40, {"B": 16, "r": 256, "M": 256, "V": 3000}),
                                         (1, 113, {"B": 16, "r": 256, "M": 256, "V": 3000}),
                                         (1, 129, {"B": 5, "r": 128, "M": 128, "V": 1000})])
def test_latent_parity(wl_id, N, over, path):
    inp, xh = _latent_case(wl_id, N, **over)
    d = _dev(inp, path)
    lat = torch.empty(N, inp.wl.B - 1, inp.wl.r, dtype=torch.bfloat16, device="cuda")
    xpress.latent_pass(d.w, upload.tokens(inp.blk), d.am1, torch.from_numpy(xh).cuda(), lat, d.ws())
    torch.cuda.synchronize()
    want = O.latent(inp, oracle_mixer(inp), xh.astype(np.float64), inp.blk, inp.am1)
    err = lat_rel_err(lat_to_f64(lat), want)
    log(f"latent {path} wl{wl_id} N={N} {over}: row-relative error {err:.2e}")
    assert err < LAT_RTOL


@pytest.mark.parametrize("path", ["table", "project"])
@pytest.mark.parametrize("N,over", [(3, {"V": 4096}), (37, {"V": 3000}), (130, {"V": 3000})])
def test_latent_fragment_order_is_the_same_values(path, N, over):
    """The latent written in the readout's fragment order holds exactly the values of the
    row-major latent, permuted (the order a step keeps lat in); 3 and 37 blocks leave a partial
    last 32-row tile, 130 blocks run the three-kernel path."""
    inp, xh = _latent_case(3 if N == 3 else 1, N, **({} if N == 3 else {"B": 16, "r": 256, "M": 512}), **over)
    d = _dev(inp, path)
    wl = inp.wl
    blk, xh_d = upload.tokens(inp.blk), torch.from_numpy(xh).cuda()
    lat_r = xpress.lat_buffer(N, wl.B, wl.r, xpress.LAT_ROWS)
    lat_f = xpress.lat_buffer(N, wl.B, wl.r, xpress.LAT_FRAGMENTS)
    xpress.latent_pass(d.w, blk, d.am1, xh_d, lat_r, d.ws())
    xpress.latent_pass(d.w, blk, d.am1, xh_d, lat_f, d.ws(), layout=xpress.LAT_FRAGMENTS)
    torch.cuda.synchronize()
    rows = N * (wl.B - 1)
    got = lat_unpack_fragments(lat_f.view(torch.int16).cpu().numpy(), rows)
    assert np.array_equal(got, lat_r.view(torch.int16).cpu().numpy())


@pytest.mark.parametrize("path", ["table", "project"])
def test_latent_causality_bit_invariance(path):
    inp, xh = _latent_case(3, 3, V=4096)
    d = _dev(inp, path)
    xh_t = torch.from_numpy(xh).cuda()
    B = inp.wl.B
    lat0 = torch.empty(3, B - 1, inp.wl.r, dtype=torch.bfloat16, device="cuda")
    ws = d.ws()
    xpress.latent_pass(d.w, upload.tokens(inp.blk), d.am1, xh_t, lat0, ws)
    for b in (1, 5, 14):
        blk2 = inp.blk.copy()
        blk2[:, b:] = (blk2[:, b:] + 777) % inp.wl.V
        lat1 = torch.empty_like(lat0)
        xpress.latent_pass(d.w, upload.tokens(blk2), d.am1, xh_t, lat1, ws)
        torch.cuda.synchronize()
        a = lat0.view(torch.int16).cpu().numpy()
        c = lat1.view(torch.int16).cpu().numpy()
        assert np.array_equal(a[:, :b], c[:, :b])
        assert not np.array_equal(a[:, b:], c[:, b:])


@pytest.mark.parametrize("path", ["table", "project"])
def test_latent_repeat_is_bit_identical(path):
    inp, xh = _latent_case(3, 4, V=4096)
    d = _dev(inp, path)
    xh_t = torch.from_numpy(xh).cuda()
    outs = []
    ws = d.ws()
    for _ in range(3):
        lat = torch.empty(4, inp.wl.B - 1, inp.wl.r, dtype=torch.bfloat16, device="cuda")
        xpress.latent_pass(d.w, upload.tokens(inp.blk), d.am1, xh_t, lat, ws)
        outs.append(lat.view(torch.int16).cpu().numpy())
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_latent_paths_agree():
    """The two-launch latent (projected table) and the three-kernel one differ only by fp32
    rounding of the embedding projection; their bf16 latents agree within a few bf16 ulps."""
    inp, xh = _latent_case(3, 8, V=4096)
    outs = []
    for path in ("table", "project"):
        d = _dev(inp, path)
        lat = torch.empty(8, inp.wl.B - 1, inp.wl.r, dtype=torch.bfloat16, device="cuda")
        xpress.latent_pass(d.w, upload.tokens(inp.blk), d.am1, torch.from_numpy(xh).cuda(), lat,
                           d.ws())
        outs.append(lat_to_f64(lat))
    err = lat_rel_err(outs[0], outs[1])
    log(f"latent paths: row-relative difference {err:.2e}")
    assert err < 1e-2


# ----------------------------------------------------------------------------------------------
# one pass, teacher-forced; whole steps

def _oracle_pass(inp, blk_p, cand=None):
    L = oracle_mixer(inp)
    xh = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    nb, _, _, hg = O.jacobi(inp, L, xh, blk_p, K=1, stop_at_fixed_point=False, cand=cand,
                            history=True)
    return nb, hg[0]


@pytest.mark.parametrize("variant", ["tiny", "strong", "wide"])
def test_one_pass_teacher_forced(variant):
    if variant == "tiny":
        inp = synth.make_inputs(1).rounded_bf16()
    elif variant == "strong":
        inp = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=8), N=6))
    else:
        inp = synth.make_inputs(replace(synth.WORKLOADS[3], V=9000), N=3)
    d = Dev(inp)
    xh = d.xh()
    got, _ = d.one_pass(inp.blk, xh)
    want, gap = _oracle_pass(inp, inp.blk)
    assert np.array_equal(got[:, 0], inp.blk[:, 0])
    bad, exempt = compare_tokens(draft_rows(got), draft_rows(want), gap)
    log(f"one pass {variant}: mismatches {bad}, near-tie rows {exempt}")
    assert bad == 0


@pytest.mark.parametrize("path", ["table", "project"])
@pytest.mark.parametrize("variant", ["tiny", "strong"])
@pytest.mark.parametrize("init", [True, False])
def test_step_to_fixed_point_matches_oracle(variant, init, path):
    if variant == "tiny":
        inp = synth.make_inputs(1).rounded_bf16()
    else:
        inp = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=8), N=6, seed=2))
    wl = inp.wl
    B = inp.raw_L.shape[1]
    N = inp.blk.shape[0]
    d = _dev(inp, path)
    blk = upload.tokens(inp.blk)
    passes = torch.zeros(1, dtype=torch.int32, device="cuda")
    flags = xpress.STOP_AT_FIXED_POINT | (xpress.INIT_FROM_BASE if init else 0)
    K = 2 * B
    xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=K, flags=flags,
                       ws=xpress.alloc_workspace(N, B, wl.r, wl.V, 0, K), passes_run=passes)
    torch.cuda.synchronize()
    L = oracle_mixer(inp)
    xh = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    start = O.initial_block(inp.base, inp.anchor, N, B) if init else inp.blk
    want, n_pass, _, hg = O.jacobi(inp, L, xh, start, K=K, stop_at_fixed_point=True,
                                   history=True)
    got = blk.cpu().numpy()
    log(f"step {path} {variant} init={init}: passes gpu {int(passes.item())} oracle {n_pass}, "
        f"min gap {hg.min():.3g}")
    bad, exempt = end_to_end_ok(got, want, hg)
    assert bad == 0
    if exempt == 0:
        assert np.array_equal(got, want)
        assert int(passes.item()) == n_pass <= B
        seq = O.sequential_greedy(inp, L, xh, inp.anchor)
        assert np.array_equal(got, seq)


def test_step_fixed_k_runs_every_pass_and_is_deterministic():
    inp = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=8), N=6, seed=4))
    N, B = inp.blk.shape
    d = Dev(inp)
    outs = []
    for _ in range(2):
        blk = upload.tokens(inp.blk)
        passes = torch.zeros(1, dtype=torch.int32, device="cuda")
        xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=3, flags=0,
                           ws=xpress.alloc_workspace(N, B, inp.wl.r, inp.wl.V, 0, 3),
                           passes_run=passes)
        torch.cuda.synchronize()
        assert int(passes.item()) == 3
        outs.append(blk.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    L = oracle_mixer(inp)
    xh = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    start = inp.blk.copy()
    start[:, 0] = inp.anchor
    want, _, _, hg = O.jacobi(inp, L, xh, start, K=3, stop_at_fixed_point=False, history=True)
    assert end_to_end_ok(outs[0], want, hg)[0] == 0


# ----------------------------------------------------------------------------------------------
# top-C

def _select_scratch(rows, V):
    """Scratch for the selection's chunk maxima (rows x 8-aligned chunk count, 2 bytes each). Rows
    of up to 153,600 ids keep them in LDS; longer rows need this buffer for the second pass to
    re-read only the chunks that can hold an answer (without it they take the exact path)."""
    nchunk8 = ((V + 7) // 8 + 7) // 8 * 8
    return torch.empty(rows * nchunk8 * 2, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("chunk_maxima", [False, True])
# 153,600 ids: the longest row whose chunk maxima stay in LDS; 153,608 and 200,003: in the
# workspace (or the exact path without one); 524,288: the longest row of the buffered path (16-bit
# chunk indexes); 524,296: the exact path either way
@pytest.mark.parametrize("C,V", [(64, 5003), (512, 8192), (700, 700), (1, 3000), (5, 7), (40, 33),
                                 (512, 153600), (64, 153608), (512, 200003), (64, 524288),
                                 (64, 524296)])
def test_topc_prepare_exact(C, V, chunk_maxima):
    rng = np.random.default_rng(6)
    N, B, r = 3, 16, 64
    rows = N * (B - 1)
    base = (np.round(rng.standard_normal((rows, V)) * 4) / 4).astype(np.float32)  # many ties
    base[0, :] = 0.0
    base[0, 5] = -0.0
    w2 = synth.bf16_round(rng.standard_normal((V, r)).astype(np.float32))
    w = _weights_with(w2, r, B, V)
    c = min(C, V)
    cand = torch.empty(rows, c, dtype=torch.int64, device="cuda")
    base_c = torch.empty(rows, c, dtype=torch.bfloat16, device="cuda")
    w2c = torch.empty(rows, c, r, dtype=torch.bfloat16, device="cuda")
    ws = _select_scratch(rows, V) if chunk_maxima else None
    xpress.topc_prepare(w, upload.base_logits(base), N, C, cand, base_c, w2c, ws)
    torch.cuda.synchronize()
    want = O.topc_select(base, C)
    got = cand.cpu().numpy()
    assert np.array_equal(got, want)
    assert np.array_equal(base_c.float().cpu().numpy(), np.take_along_axis(base, want, axis=1))
    assert np.array_equal(w2c.float().cpu().numpy(), w2[want])


@pytest.mark.parametrize("chunk_maxima", [False, True])
@pytest.mark.parametrize("C,V", [(512, 8192), (64, 5003), (1024, 20000), (512, 160000)])
def test_topc_prepare_adversarial_rows(C, V, chunk_maxima):
    """Rows that defeat a per-thread shortlist (sorted rows, the answer concentrated in the ids one
    thread visits, very few distinct values) must still give the exact candidate sets."""
    rng = np.random.default_rng(11)
    N, B, r = 1, 8, 64
    rows = N * (B - 1)
    base = np.zeros((rows, V), dtype=np.float32)
    base[0] = np.arange(V) / V * 100                      # ascending
    base[1] = base[0][::-1]                               # descending
    chunks = np.arange((V + 7) // 8)
    ids7 = (8 * chunks[chunks % 256 == 7][:, None] + np.arange(8)[None, :]).reshape(-1)
    ids7 = ids7[ids7 < V]
    base[2, ids7] = 1.0 + np.arange(ids7.size) % 37       # best values all in one thread's ids
    base[3] = rng.integers(0, 3, V)                       # three distinct values
    base[4] = np.round(rng.standard_normal(V) * 2) / 2
    base[4, rng.choice(V, 40, replace=False)] = 50.0      # a few large values
    base[5] = -1.0                                        # all equal
    base[6] = rng.standard_normal(V)
    base = synth.bf16_round(base)
    w2 = synth.bf16_round(rng.standard_normal((V, r)).astype(np.float32))
    w = _weights_with(w2, r, B, V)
    c = min(C, V)
    cand = torch.empty(rows, c, dtype=torch.int64, device="cuda")
    base_c = torch.empty(rows, c, dtype=torch.bfloat16, device="cuda")
    w2c = torch.empty(rows, c, r, dtype=torch.bfloat16, device="cuda")
    ws = _select_scratch(rows, V) if chunk_maxima else None
    xpress.topc_prepare(w, upload.base_logits(base), N, C, cand, base_c, w2c, ws)
    torch.cuda.synchronize()
    want = O.topc_select(base, C)
    got = cand.cpu().numpy()
    for i in range(rows):
        assert np.array_equal(got[i], want[i]), f"row {i}"
    assert np.array_equal(base_c.float().cpu().numpy(), np.take_along_axis(base, want, axis=1))


# gathered: rows from w2c; ids: rows from w2 through cand (the step's form; topc_prepare then
# skips the gather). C = 96 and 100 at r = 256: whole and ragged last rounds of both forms.
@pytest.mark.parametrize("form", ["gathered", "ids"])
@pytest.mark.parametrize("r,C", [(256, 96), (256, 100), (128, 300), (64, 37)])
def test_topc_readout_dyadic_exact_and_membership(form, r, C):
    rng = np.random.default_rng(7)
    N, B, V = 4, 16, 6000
    lat, w2, base = _readout_case(8, N, B, r, V)
    w = _weights_with(w2, r, B, V)
    rows = N * (B - 1)
    cand = torch.empty(rows, C, dtype=torch.int64, device="cuda")
    base_c = torch.empty(rows, C, dtype=torch.bfloat16, device="cuda")
    w2c = torch.empty(rows, C, r, dtype=torch.bfloat16, device="cuda") if form == "gathered" else None
    xpress.topc_prepare(w, upload.base_logits(base), N, C, cand, base_c, w2c)
    blk0 = rng.integers(0, V, (N, B))
    blk = upload.tokens(blk0)
    log(f"top-C readout {form} r={r} C={C}")
    if form == "gathered":
        xpress.readout_argmax_topc(upload.bf16_tensor(lat), w2c, base_c, cand, blk)
    else:
        xpress.readout_argmax_topc_ids(w, upload.bf16_tensor(lat), base_c, cand, blk)
    torch.cuda.synchronize()
    cand_o = O.topc_select(base, C)
    best, gap, _ = O.readout_argmax(lat, w2, base, cand=cand_o)
    got = draft_rows(blk.cpu().numpy())
    assert np.array_equal(got, best)
    for p in range(rows):
        assert got[p] in cand_o[p]


@pytest.mark.parametrize("form", ["gathered", "ids"])
def test_topc_readout_ties_go_to_the_lowest_id_whatever_the_candidate_order(form):
    """Each row's candidates handed over in a seeded shuffled order (with base_c and the gathered
    rows permuted alike): the winner is the same lowest-id winner as with ascending candidates
    (qwen3_xpress page: the candidate set is only indexed, so its order does not matter). The
    dyadic case plants exact top ties between a low and a high id."""
    rng = np.random.default_rng(13)
    N, B, V, r, C = 4, 16, 6000, 256, 96
    lat, w2, base = _readout_case(8, N, B, r, V)
    w = _weights_with(w2, r, B, V)
    rows = N * (B - 1)
    cand_o = O.topc_select(base, C)
    perm = np.argsort(rng.random((rows, C)), axis=1)
    perm[0] = np.arange(C)[::-1]  # fully descending on one row
    cand_s = np.take_along_axis(cand_o, perm, axis=1)
    base_c_s = np.take_along_axis(base, cand_s, axis=1)
    cand = upload.tokens(cand_s)
    base_c = upload.bf16_tensor(base_c_s)
    blk = upload.tokens(rng.integers(0, V, (N, B)))
    log(f"top-C readout {form}, shuffled candidates")
    if form == "gathered":
        w2c = upload.bf16_tensor(w2[cand_s])
        xpress.readout_argmax_topc(upload.bf16_tensor(lat), w2c, base_c, cand, blk)
    else:
        xpress.readout_argmax_topc_ids(w, upload.bf16_tensor(lat), base_c, cand, blk)
    torch.cuda.synchronize()
    best, _, _ = O.readout_argmax(lat, w2, base, cand=cand_o)
    best_s, _, _ = O.readout_argmax(lat, w2, base, cand=cand_s)
    assert np.array_equal(best, best_s)  # the oracle's rule is order-free too
    got = draft_rows(blk.cpu().numpy())
    assert np.array_equal(got, best)
    planted = [p for p in range(0, rows, 3) if best[p] == p]
    assert len(planted) >= rows // 6  # the planted low ids do win their ties


@pytest.mark.parametrize("chunk_maxima", [False, True])
@pytest.mark.parametrize("V,C", [(5003, 64), (151936, 512)])
def test_topc_rows_with_fewer_finite_values_than_candidates(V, C, chunk_maxima):
    """Rows where fewer than C values are finite (the rest -inf, as a vocabulary mask leaves
    them): the candidate sets are still the C largest under (value desc, id asc) -- -inf below
    every finite value, ties to the lowest ids -- so every id is in range, and the top-C readout
    and the step's starting block pick candidates. Inputs that are not finite fall outside the
    pages' method; this checks that the selection stays exact and in range for them."""
    rng = np.random.default_rng(14)
    N, B, r = 2, 3, 64
    rows = N * (B - 1)
    base = synth.bf16_round(rng.standard_normal((rows, V)).astype(np.float32))
    base[0, :] = -np.inf
    base[0, rng.choice(V, C // 4, replace=False)] = 1.5         # C/4 finite values, tied
    base[1, :] = -np.inf                                        # no finite value at all
    base[2, :] = -np.inf
    keep = rng.choice(V, C - 1, replace=False)
    base[2, keep] = synth.bf16_round(rng.standard_normal(C - 1).astype(np.float32))
    base[3, rng.choice(V, V // 2, replace=False)] = -np.inf     # plenty of finite values left
    w2 = synth.bf16_round(rng.standard_normal((V, r)).astype(np.float32) * 0.1)
    w = _weights_with(w2, r, B, V)
    cand = torch.empty(rows, C, dtype=torch.int64, device="cuda")
    base_c = torch.empty(rows, C, dtype=torch.bfloat16, device="cuda")
    ws = _select_scratch(rows, V) if chunk_maxima else None
    log(f"top-C prepare with -inf rows V={V} C={C} chunk_maxima={chunk_maxima}")
    xpress.topc_prepare(w, upload.base_logits(base), N, C, cand, base_c, None, ws)
    torch.cuda.synchronize()
    got = cand.cpu().numpy()
    assert got.min() >= 0 and got.max() < V
    want = O.topc_select(base, C)
    assert np.array_equal(got, want)
    assert np.array_equal(base_c.float().cpu().numpy(), np.take_along_axis(base, want, axis=1))
    lat = synth.bf16_round(rng.standard_normal((rows, r)).astype(np.float32))
    blk = upload.tokens(np.zeros((N, B), np.int64))
    xpress.readout_argmax_topc_ids(w, upload.bf16_tensor(lat), base_c, cand, blk)
    torch.cuda.synchronize()
    best, gap, _ = O.readout_argmax(lat, w2, base, cand=want)
    got_t = draft_rows(blk.cpu().numpy())
    assert all(got_t[p] in want[p] for p in range(rows))
    assert compare_tokens(got_t, best, gap)[0] == 0
    assert got_t[1] == 0  # every logit -inf: the lowest id


@pytest.mark.parametrize("C", [1, 10 ** 6])
def test_topc_step_limits(C):
    """C = 1 always returns argmax(base); C >= V scores every id, as the full-vocabulary step."""
    inp = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=8), N=4, seed=5))
    N, B = inp.blk.shape
    wl = inp.wl
    d = Dev(inp)
    blk = upload.tokens(inp.blk)
    xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=4, C=C,
                       flags=xpress.INIT_FROM_BASE,
                       ws=xpress.alloc_workspace(N, B, wl.r, wl.V, C, 4))
    torch.cuda.synchronize()
    got = blk.cpu().numpy()
    if C == 1:
        assert np.array_equal(draft_rows(got), np.argmax(inp.base, axis=1))
        return
    L = oracle_mixer(inp)
    xh = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    start = O.initial_block(inp.base, inp.anchor, N, B)
    want, _, _, hg = O.jacobi(inp, L, xh, start, K=4, stop_at_fixed_point=False, history=True)
    assert end_to_end_ok(got, want, hg)[0] == 0


@pytest.mark.parametrize("path,M,r", [("table", 128, 64), ("project", 128, 64), ("table", 1024, 64),
                                      ("table", 512, 256), ("project", 512, 256)])
def test_topc_step_matches_oracle(path, M, r):
    """With the projected table the top-C readout sums the latent shares itself (no lat); at
    M = 1024 there are 16 slice shares, two rounds of eight; r = 256 with M = 512 is the shape of
    the 32-block top-512 workload."""
    inp = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=8, M=M, r=r), N=6, seed=6))
    N, B = inp.blk.shape
    wl = inp.wl
    C = 48
    d = _dev(inp, path)
    blk = upload.tokens(inp.blk)
    passes = torch.zeros(1, dtype=torch.int32, device="cuda")
    xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=2 * B, C=C,
                       flags=xpress.INIT_FROM_BASE | xpress.STOP_AT_FIXED_POINT,
                       ws=xpress.alloc_workspace(N, B, wl.r, wl.V, C, 2 * B), passes_run=passes)
    torch.cuda.synchronize()
    L = oracle_mixer(inp)
    xh = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    cand = O.topc_select(inp.base, C)
    start = O.initial_block(inp.base, inp.anchor, N, B)
    want, n_pass, _, hg = O.jacobi(inp, L, xh, start, K=2 * B, stop_at_fixed_point=True,
                                   cand=cand, history=True)
    got = blk.cpu().numpy()
    bad, exempt = end_to_end_ok(got, want, hg)
    assert bad == 0
    if exempt == 0:
        assert int(passes.item()) == n_pass
    for p, tok in enumerate(draft_rows(got)):
        assert tok in cand[p]


# B = 2: one draft slot per block (slot 1 reads the anchor; rows = N); B = 16 at r = 128 with a
# ragged V, K > B; each with and without candidates, on both latent paths
@pytest.mark.parametrize("path", ["table", "project"])
@pytest.mark.parametrize("B,r,V,N,C", [(2, 64, 1001, 5, 0), (2, 64, 1001, 5, 7),
                                       (16, 128, 3001, 3, 0), (16, 128, 3001, 3, 100)])
def test_step_edge_shapes(B, r, V, N, C, path):
    inp = strong(synth.make_inputs(replace(synth.WORKLOADS[1], B=B, r=r, V=V), N=N, seed=9))
    wl = inp.wl
    K = 2 * B + 1
    d = _dev(inp, path)
    blk = upload.tokens(inp.blk)
    passes = torch.zeros(1, dtype=torch.int32, device="cuda")
    log(f"step edge shape B={B} r={r} V={V} N={N} C={C} {path}")
    xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=K, C=C,
                       flags=xpress.INIT_FROM_BASE | xpress.STOP_AT_FIXED_POINT,
                       ws=xpress.alloc_workspace(N, B, r, V, C, K), passes_run=passes)
    torch.cuda.synchronize()
    L = oracle_mixer(inp)
    xh = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    cand = O.topc_select(inp.base, C) if C else None
    start = O.initial_block(inp.base, inp.anchor, N, B)
    want, n_pass, _, hg = O.jacobi(inp, L, xh, start, K=K, stop_at_fixed_point=True, cand=cand,
                                   history=True)
    got = blk.cpu().numpy()
    bad, exempt = end_to_end_ok(got, want, hg)
    log(f"  passes gpu {int(passes.item())} oracle {n_pass}, exempt rows {exempt}")
    assert bad == 0
    assert np.array_equal(got[:, 0], inp.anchor)
    if exempt == 0:
        assert np.array_equal(got, want)
        assert int(passes.item()) == n_pass
    if C:
        assert all(got[n, b] in cand[n * (B - 1) + b - 1] for n in range(N) for b in range(1, B))


@pytest.mark.parametrize("path", ["table", "project"])
def test_step_at_40_blocks_matches_oracle(path):
    """A 15-pass step at 40 blocks of the 32-block workload's shape (r = 256, M = 512; V = 3000):
    on the table path 320 share workgroups, two per CU; on either path the drafts agree with the
    oracle on every block up to near ties (end-to-end rule)."""
    inp = synth.make_inputs(replace(synth.WORKLOADS[3], V=3000), N=40, seed=4).rounded_bf16()
    wl = inp.wl
    K = 15
    d = _dev(inp, path)
    blk = torch.zeros(wl.N, wl.B, dtype=torch.int64, device="cuda")
    log(f"40-block step, {path}")
    xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=K, flags=xpress.INIT_FROM_BASE,
                       ws=xpress.alloc_workspace(wl.N, wl.B, wl.r, wl.V, 0, K))
    torch.cuda.synchronize()
    L = oracle_mixer(inp)
    xh = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    start = O.initial_block(inp.base, inp.anchor, wl.N, wl.B)
    want, _, _, hg = O.jacobi(inp, L, xh, start, K=K, stop_at_fixed_point=False, history=True)
    got = blk.cpu().numpy()
    bad, exempt = end_to_end_ok(got, want, hg)
    log(f"  disallowed mismatches {bad}, near-tie row-passes {exempt}")
    assert bad == 0
    assert np.array_equal(got[:, 0], inp.anchor)


@pytest.mark.parametrize("C,path", [(0, "table"), (0, "project"), (40, "table")])
def test_step_is_block_permutation_equivariant(C, path):
    """Blocks never mix: permuting the blocks of every per-block input (h, the base rows, anchor,
    am1) permutes the step's drafts and leaves the pass count, bit for bit."""
    inp = synth.make_inputs(replace(synth.WORKLOADS[3], V=2000), N=9, seed=6).rounded_bf16()
    wl = inp.wl
    perm = np.random.default_rng(1).permutation(wl.N)
    rows = (perm[:, None] * (wl.B - 1) + np.arange(wl.B - 1)[None, :]).reshape(-1)
    pinp = replace(inp, h=inp.h[perm], base=inp.base[rows], blk=inp.blk[perm], am1=inp.am1[perm])
    K = 15
    outs = []
    for x in (inp, pinp):
        d = _dev(x, path)
        blk = torch.zeros(wl.N, wl.B, dtype=torch.int64, device="cuda")
        passes = torch.zeros(1, dtype=torch.int32, device="cuda")
        xpress.jacobi_step(d.w, d.h, d.base, d.anchor, d.am1, blk, K=K, C=C,
                           flags=xpress.INIT_FROM_BASE | xpress.STOP_AT_FIXED_POINT,
                           ws=xpress.alloc_workspace(wl.N, wl.B, wl.r, wl.V, C, K),
                           passes_run=passes)
        torch.cuda.synchronize()
        outs.append((blk.cpu().numpy(), int(passes.item())))
    (got, p0), (pgot, p1) = outs
    log(f"permutation equivariance C={C} {path}: passes {p0} / {p1}")
    assert np.array_equal(pgot, got[perm])
    assert p0 == p1
