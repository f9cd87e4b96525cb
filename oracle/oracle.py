"""NumPy-facing wrapper of the plain C oracle of the XPress Jacobi refinement pass.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. It loads ``liboracle.so`` built from
``xpress_oracle.c`` with gcc (no HIP, nothing shared with the device library) and only marshals
arguments: every step of the method runs in the C code, in double precision.

Parity pins of each function live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "xpress_oracle.c"
LIB = HERE / "liboracle.so"

_lib = None


def build(force: bool = False) -> Path:
    """Compile the oracle with gcc (plain -O2, no fast-math, no FMA contraction, OpenMP)."""
    if force or not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
        tmp = LIB.with_suffix(f".so.tmp{os.getpid()}")
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", str(SRC), "-o", str(tmp), "-lm"],
            check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(str(LIB))
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        lib.xo_set_threads.argtypes = [i32]
        lib.xo_max_threads.restype = i32
        lib.xo_fold_mixer.argtypes = [P, i32, i32, P]
        lib.xo_hidden_cache.argtypes = [P, P, P, P, i32, i32, i32, i32, P]
        lib.xo_initial_block.argtypes = [P, i64, P, i32, i32, i64, P]
        lib.xo_topc_select.argtypes = [P, i64, i64, i64, i32, P]
        lib.xo_latent.argtypes = [P, P, P, P, P, P, i32, i32, i32, i64, P, P, P, i32, P, P]
        lib.xo_readout_argmax.argtypes = [P, P, P, i64, i64, i64, i32, P, P, P]
        lib.xo_readout_argmax_topc.argtypes = [P, P, P, i64, P, i64, i32, i32, P, P, P]
        lib.xo_jacobi.restype = i32
        lib.xo_jacobi.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i64, P, P, i64, P, i32, P,
                                  i32, i32, i32, P, P, P]
        lib.xo_sequential_greedy.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i64, P, P, i64,
                                             P, P, i32, P, i32, P, P]
        _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    _load().xo_set_threads(int(n))


def max_threads() -> int:
    return int(_load().xo_max_threads())


def fold_mixer(raw_L: np.ndarray) -> np.ndarray:
    """Folded per-channel mixer L = raw * tril + I, [r, B, B] float64."""
    raw = _f32(raw_L)
    r, B, _ = raw.shape
    out = np.empty((r, B, B), dtype=np.float64)
    _load().xo_fold_mixer(_p(raw), r, B, _p(out))
    return out


def hidden_cache(h, down_h, down_g, in_proj) -> np.ndarray:
    """xh [N, B, r] float64: the hidden half of in_proj applied to [down_h(h) ++ down_g(mean h)]."""
    h, dh, dg, pr = _f32(h), _f32(down_h), _f32(down_g), _f32(in_proj)
    N, B, H = h.shape
    r = dh.shape[0]
    assert dh.shape == (r, H) and dg.shape == (r, H) and pr.shape == (r, 3 * r)
    out = np.empty((N, B, r), dtype=np.float64)
    _load().xo_hidden_cache(_p(h), _p(dh), _p(dg), _p(pr), N, B, H, r, _p(out))
    return out


def initial_block(base, anchor, N: int, B: int) -> np.ndarray:
    base, anchor = _f32(base), _i64(anchor)
    rows, V = base.shape
    assert rows == N * (B - 1)
    out = np.empty((N, B), dtype=np.int64)
    _load().xo_initial_block(_p(base), V, _p(anchor), N, B, V, _p(out))
    return out


def topc_select(base, C: int) -> np.ndarray:
    """[rows, min(C, V)] candidate ids, ascending, chosen by (value desc, id asc)."""
    base = _f32(base)
    rows, V = base.shape
    c = min(C, V)
    out = np.empty((rows, c), dtype=np.int64)
    _load().xo_topc_select(_p(base), V, rows, V, C, _p(out))
    return out


def latent(inp, L, xh, blk, am1, *, return_u: bool = False):
    """lat [N, B-1, r] float64 (and the mixer output u [N, B, r] when asked)."""
    w1, pr, wg, wu, wd = (_f32(inp.w1), _f32(inp.in_proj), _f32(inp.w_gate), _f32(inp.w_up),
                          _f32(inp.w_down))
    L, xh, blk, am1 = _f64(L), _f64(xh), _i64(blk), _i64(am1)
    N, B = blk.shape
    V, r = w1.shape
    M = wg.shape[0]
    lat = np.empty((N, B - 1, r), dtype=np.float64)
    u = np.empty((N, B, r), dtype=np.float64) if return_u else None
    _load().xo_latent(_p(w1), _p(pr), _p(L), _p(wg), _p(wu), _p(wd), B, r, M, V, _p(blk),
                      _p(am1), _p(xh), N, _p(lat), _p(u))
    return (lat, u) if return_u else lat


def readout_argmax(lat, w2, base, *, cand=None):
    """(best ids [rows] int64, gap [rows], best logit [rows]) of base + lat . w2^T.

    With ``cand`` ([rows, c] vocab ids) only the candidates are scored.
    """
    lat, w2, base = _f64(lat), _f32(w2), _f32(base)
    rows, r = lat.shape
    V = w2.shape[0]
    assert base.shape[0] == rows
    best = np.empty(rows, dtype=np.int64)
    gap = np.empty(rows, dtype=np.float64)
    val = np.empty(rows, dtype=np.float64)
    ld = base.shape[1]
    if cand is None:
        assert base.shape[1] == V
        _load().xo_readout_argmax(_p(lat), _p(w2), _p(base), ld, rows, V, r, _p(best), _p(gap),
                                  _p(val))
    else:
        cand = _i64(cand)
        c = cand.shape[1]
        _load().xo_readout_argmax_topc(_p(lat), _p(w2), _p(base), ld, _p(cand), rows, c, r,
                                       _p(best), _p(gap), _p(val))
    return best, gap, val


def jacobi(inp, L, xh, blk0, *, K: int, stop_at_fixed_point: bool, cand=None,
           history: bool = False):
    """Run Jacobi passes from ``blk0``. Returns (blk, passes, hist_blk, hist_gap)."""
    w1, pr, wg, wu, wd, w2 = (_f32(inp.w1), _f32(inp.in_proj), _f32(inp.w_gate),
                              _f32(inp.w_up), _f32(inp.w_down), _f32(inp.w2))
    base = _f32(inp.base)
    L, xh = _f64(L), _f64(xh)
    blk = _i64(blk0).copy()
    am1 = _i64(inp.am1)
    N, B = blk.shape
    V, r = w1.shape
    M = wg.shape[0]
    rows = N * (B - 1)
    hb = np.empty((K + 1, N, B), dtype=np.int64) if history else None
    hg = np.empty((K, rows), dtype=np.float64) if history else None
    c = 0
    if cand is not None:
        cand = _i64(cand)
        c = cand.shape[1]
    passes = _load().xo_jacobi(_p(w1), _p(pr), _p(L), _p(wg), _p(wu), _p(wd), _p(w2), B, r, M,
                               V, _p(xh), _p(base), base.shape[1], _p(am1), N, _p(cand), c, K,
                               int(stop_at_fixed_point), _p(blk), _p(hb), _p(hg))
    if history:
        hb, hg = hb[: passes + 1], hg[:passes]
    return blk, int(passes), hb, hg


def sequential_greedy(inp, L, xh, anchor, *, cand=None, filler=None) -> np.ndarray:
    """Slot-by-slot greedy decode by brute force, [N, B] (column 0 is the anchor)."""
    w1, pr, wg, wu, wd, w2 = (_f32(inp.w1), _f32(inp.in_proj), _f32(inp.w_gate),
                              _f32(inp.w_up), _f32(inp.w_down), _f32(inp.w2))
    base = _f32(inp.base)
    L, xh = _f64(L), _f64(xh)
    anchor, am1 = _i64(anchor), _i64(inp.am1)
    N = anchor.shape[0]
    V, r = w1.shape
    B = L.shape[1]
    M = wg.shape[0]
    if filler is None:
        filler = np.zeros((N, B), dtype=np.int64)
    filler = _i64(filler)
    c = 0
    if cand is not None:
        cand = _i64(cand)
        c = cand.shape[1]
    out = np.empty((N, B), dtype=np.int64)
    _load().xo_sequential_greedy(_p(w1), _p(pr), _p(L), _p(wg), _p(wu), _p(wd), _p(w2), B, r,
                                 M, V, _p(xh), _p(base), base.shape[1], _p(anchor), _p(am1), N,
                                 _p(cand), c, _p(filler), _p(out))
    return out
