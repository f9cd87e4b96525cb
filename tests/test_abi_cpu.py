"""The C-ABI library without a GPU: it loads, exports every declared entry point, and rejects bad
arguments on the host (no kernel is launched by any call here)."""
import ctypes
import subprocess

import pytest

from jacobi_block_refiner_amd import xpress


def test_library_exports_every_declared_symbol():
    names = xpress.declared_symbols()
    assert len(names) >= 10
    L = xpress.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", str(xpress.LIB_PATH)], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_workspace_size_grows_with_blocks_and_candidates():
    a = xpress.workspace_size(256, 16, 256, 151936, 0, 15)
    b = xpress.workspace_size(512, 16, 256, 151936, 0, 15)
    c = xpress.workspace_size(256, 16, 256, 151936, 512, 15)
    assert 0 < a < b
    # top-C adds cand (int64) + base_c (bf16) per candidate and drops the full-vocabulary readout's
    # partials (256 per row); the passes read w2 through the ids, so no gathered [rows, C, r] copy
    # (1 GB here), and rows of 151,936 ids keep the selection's chunk maxima in LDS. (At 256
    # blocks the layout of n_max itself is the largest, so the regions add up exactly.)
    rows = 256 * 15
    part = rows * 256 * 8
    assert a - part + rows * 512 * (8 + 2) <= c < a - part + rows * 512 * (8 + 2) + 4096
    # rows of more than 153,600 ids keep the chunk maxima (2 bytes per 8 ids, 8-chunk groups) in
    # the workspace
    V = 200003
    nchunk8 = ((V + 7) // 8 + 7) // 8 * 8
    full = xpress.workspace_size(256, 16, 256, V, 0, 15)
    top = xpress.workspace_size(256, 16, 256, V, 512, 15)
    assert top >= full - part + rows * 512 * (8 + 2) + rows * nchunk8 * 2


@pytest.mark.parametrize("B,r,V", [(1, 256, 1000), (17, 256, 1000), (16, 96, 1000),
                                   (16, 256, 0), (16, 256, 1 << 24)])
def test_bad_shapes_are_rejected(B, r, V):
    out = ctypes.c_size_t()
    st = xpress.lib().xpress_workspace_size(4, B, r, V, 0, 1, ctypes.byref(out))
    assert st == xpress.ERR_ARG
    assert xpress.lib().xpress_last_error()


def test_null_weights_and_pointers_are_rejected():
    L = xpress.lib()
    st = L.xpress_latent_pass(None, None, None, None, 4, None, 0, None, 0, None)
    assert st == xpress.ERR_ARG and b"NULL" in L.xpress_last_error()
    w = xpress._Weights(B=16, r=256, H=4096, M=512, V=151936)
    st = L.xpress_jacobi_step(ctypes.byref(w), None, None, 151936, None, None, 4, 15, 0, 1, None,
                              None, None, 0, None)
    assert st == xpress.ERR_ARG
    st = L.xpress_fold_mixer(None, 256, 16, None, None)
    assert st == xpress.ERR_ARG


def test_n_zero_is_a_noop_and_unknown_flags_are_rejected():
    L = xpress.lib()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced
    w = xpress._Weights(B=16, r=256, H=4096, M=512, V=151936, w1=fake, down_h=fake,
                        down_g=fake, in_proj=fake, mix_L=fake, w_gate=fake, w_up=fake,
                        w_down=fake, w2=fake)
    assert L.xpress_latent_pass(ctypes.byref(w), fake, fake, fake, 0, fake, 0, fake, 0, None) == xpress.OK
    st = L.xpress_jacobi_step(ctypes.byref(w), fake, fake, 151936, fake, fake, 4, 15, 0, 0x10,
                              fake, None, fake, 1 << 30, None)
    assert st == xpress.ERR_ARG and b"flag" in L.xpress_last_error()


def test_small_workspace_and_bad_stride_are_rejected():
    L = xpress.lib()
    fake = ctypes.c_void_p(1 << 20)
    w = xpress._Weights(B=16, r=256, H=4096, M=512, V=151936, w1=fake, down_h=fake,
                        down_g=fake, in_proj=fake, mix_L=fake, w_gate=fake, w_up=fake,
                        w_down=fake, w2=fake)
    st = L.xpress_readout_argmax(ctypes.byref(w), fake, 0, fake, 151936, 4, fake, None, fake, 16,
                                 None)
    assert st == xpress.ERR_WORKSPACE
    st = L.xpress_readout_argmax(ctypes.byref(w), fake, 0, fake, 151937, 4, fake, None, fake,
                                 1 << 30, None)
    assert st == xpress.ERR_ARG
    st = L.xpress_readout_argmax(ctypes.byref(w), fake, 2, fake, 151936, 4, fake, None, fake,
                                 1 << 30, None)
    assert st == xpress.ERR_ARG and b"lat_layout" in L.xpress_last_error()
    misaligned = ctypes.c_void_p((1 << 20) + 2)
    st = L.xpress_readout_argmax(ctypes.byref(w), misaligned, 0, fake, 151936, 4, fake, None, fake,
                                 1 << 30, None)
    assert st == xpress.ERR_ARG and b"aligned" in L.xpress_last_error()
    # a base row stride past 2^27 elements is refused (the readout's 32-bit copy offsets)
    for ld in ((1 << 27) + 8, 1 << 28):
        st = L.xpress_readout_argmax(ctypes.byref(w), fake, 0, fake, ld, 4, fake, None, fake,
                                     1 << 30, None)
        assert st == xpress.ERR_ARG and b"base_ld" in L.xpress_last_error()


def test_fold_embedding_and_table_arguments_are_checked():
    L = xpress.lib()
    fake = ctypes.c_void_p(1 << 20)
    w = xpress._Weights(B=16, r=256, H=4096, M=512, V=151936, w1=fake, down_h=fake,
                        down_g=fake, in_proj=fake, mix_L=fake, w_gate=fake, w_up=fake,
                        w_down=fake, w2=fake)
    assert L.xpress_fold_embedding(None, fake, None) == xpress.ERR_ARG
    assert L.xpress_fold_embedding(ctypes.byref(w), None, None) == xpress.ERR_ARG
    assert L.xpress_fold_embedding(ctypes.byref(w), ctypes.c_void_p((1 << 20) + 4),
                                   None) == xpress.ERR_ARG
    bad = xpress._Weights(B=16, r=96, H=4096, M=512, V=151936, w1=fake, in_proj=fake)
    assert L.xpress_fold_embedding(ctypes.byref(bad), fake, None) == xpress.ERR_ARG
    # a misaligned projected table is rejected before anything is enqueued
    w.w1p = (1 << 20) + 8
    st = L.xpress_latent_pass(ctypes.byref(w), fake, fake, fake, 4, fake, 0, fake, 1 << 30, None)
    assert st == xpress.ERR_ARG and b"w1p" in L.xpress_last_error()
    # with the table, the latent scratch holds the M/64 slice shares of every block
    w.w1p = 1 << 20
    st = L.xpress_latent_pass(ctypes.byref(w), fake, fake, fake, 4, fake, 0, fake, 1024, None)
    assert st == xpress.ERR_WORKSPACE
    st = L.xpress_latent_pass(ctypes.byref(w), fake, fake, fake, 4, fake, 7, fake, 1 << 30, None)
    assert st == xpress.ERR_ARG and b"lat_layout" in L.xpress_last_error()


def test_workspace_for_n_max_fits_every_smaller_n():
    """A workspace sized for n_max covers every N <= n_max (the table path's latent scratch makes
    the size non-monotone in N where its slices widen from 32 to 64 units and where that path
    stops: N * M/64 = 448 share workgroups, i.e. after 28, 56, 112, 224 or 448 blocks depending
    on M)."""
    for n_max in (15, 16, 17, 28, 29, 31, 32, 33, 56, 57, 64, 65, 96, 112, 113, 128, 160, 224,
                  225, 256, 257, 448, 449):
        big = xpress.workspace_size(n_max, 16, 256, 151936, 0, 15)
        for n in (1, 8, 9, 16, 17, 28, 29, 32, 33, 56, 57, 64, 65, 96, 112, 113, 128, 129, 224,
                  225, 256, 448, 449, n_max):
            if n <= n_max:
                assert xpress.workspace_size(n, 16, 256, 151936, 0, 15) <= big, (n, n_max)


@pytest.mark.parametrize("V,rows,want", [(151936, 15, 256), (151936, 512, 256), (151936, 513, 128),
                                         (151936, 1536, 80), (151936, 3840, 32),
                                         (151936, 20000, 8), (100, 3840, 4), (33, 1, 2),
                                         (5003, 600, 128)])
def test_readout_range_count(V, rows, want):
    """Partials per readout row: 256 ranges (at most ceil(V/32)) up to one 512-row chunk, about
    256 / chunks beyond, a multiple of 8 and at least 8 (host-side arithmetic, no kernel)."""
    assert xpress.readout_tiles(V, rows) == want


def test_readout_range_count_rejects_bad_arguments():
    L = xpress.lib()
    out = ctypes.c_int32()
    assert L.xpress_readout_tiles(151936, 0, ctypes.byref(out)) == xpress.ERR_ARG
    assert L.xpress_readout_tiles(0, 15, ctypes.byref(out)) == xpress.ERR_ARG
    assert L.xpress_readout_tiles(151936, 15, None) == xpress.ERR_ARG


def test_topc_ids_readout_arguments_are_checked():
    L = xpress.lib()
    fake = ctypes.c_void_p(1 << 20)
    w = xpress._Weights(B=16, r=256, H=4096, M=512, V=151936, w2=fake)
    assert L.xpress_readout_argmax_topc_ids(None, fake, fake, fake, 4, 512, fake, None,
                                            None) == xpress.ERR_ARG
    assert L.xpress_readout_argmax_topc_ids(ctypes.byref(w), fake, fake, fake, 4, 151937, fake,
                                            None, None) == xpress.ERR_ARG
    assert L.xpress_readout_argmax_topc_ids(ctypes.byref(w), fake, None, fake, 4, 512, fake, None,
                                            None) == xpress.ERR_ARG
    assert L.xpress_readout_argmax_topc_ids(ctypes.byref(w), fake, fake, fake, 0, 512, fake, None,
                                            None) == xpress.OK
    misaligned = ctypes.c_void_p((1 << 20) + 2)
    st = L.xpress_topc_prepare(ctypes.byref(w), fake, 151936, 4, 512, fake, fake, misaligned,
                               None, 0, None)
    assert st == xpress.ERR_ARG and b"w2c" in L.xpress_last_error()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library every entry point raises."""
    monkeypatch.setattr(xpress, "LIB_PATH", tmp_path / "libxpress.so")
    monkeypatch.setattr(xpress, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        xpress.readout_tiles(151936, 480)
    with pytest.raises(RuntimeError, match="missing"):
        xpress.lib()
