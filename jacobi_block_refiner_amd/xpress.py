"""Thin ctypes binding of ``libxpress.so`` (the C ABI in ``include/xpress.h``).

Argument marshalling only: tensors are passed as device pointers together with the current HIP
stream of PyTorch, and every step of the method runs in the library's HIP kernels. There is no
fallback: if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import re
from dataclasses import dataclass
from pathlib import Path

import torch

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libxpress.so"
HEADER = PKG.parent / "include" / "xpress.h"

OK, ERR_ARG, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3
LAT_ROWS, LAT_FRAGMENTS = 0, 1
INIT_FROM_BASE = 1
STOP_AT_FIXED_POINT = 2


class XpressError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"xpress status {status}: {message}")
        self.status = status


class _Weights(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("r", ctypes.c_int32), ("H", ctypes.c_int32),
        ("M", ctypes.c_int32), ("V", ctypes.c_int64),
        ("w1", ctypes.c_void_p), ("down_h", ctypes.c_void_p), ("down_g", ctypes.c_void_p),
        ("in_proj", ctypes.c_void_p), ("mix_L", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
        ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p), ("w2", ctypes.c_void_p),
        ("w1p", ctypes.c_void_p),
    ]


_lib = None


def declared_symbols() -> list[str]:
    """Function names declared in include/xpress.h."""
    text = HEADER.read_text()
    return re.findall(r"^(?:xpress_status|const char\*)\s+(xpress_\w+)\(", text, flags=re.M)


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with jacobi_block_refiner_amd.build.build()")
        L = ctypes.CDLL(str(LIB_PATH))
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        W = ctypes.POINTER(_Weights)
        sig = {
            "xpress_workspace_size": [i32, i32, i32, i64, i32, i32, ctypes.POINTER(sz)],
            "xpress_fold_mixer": [P, i32, i32, P, P],
            "xpress_fold_embedding": [W, P, P],
            "xpress_hidden_cache": [W, P, i32, P, P, sz, P],
            "xpress_initial_block": [P, i64, P, i32, i32, i64, P, P],
            "xpress_latent_pass": [W, P, P, P, i32, P, ctypes.c_uint32, P, sz, P],
            "xpress_readout_argmax": [W, P, ctypes.c_uint32, P, i64, i32, P, P, P, sz, P],
            "xpress_readout_tiles": [i64, i32, ctypes.POINTER(i32)],
            "xpress_readout_partials": [W, P, ctypes.c_uint32, P, i64, i32, P, P],
            "xpress_argmax_reduce": [P, i32, i32, i32, P, P, P],
            "xpress_topc_prepare": [W, P, i64, i32, i32, P, P, P, P, sz, P],
            "xpress_readout_argmax_topc": [P, P, P, P, i32, i32, i32, i32, P, P, P],
            "xpress_readout_argmax_topc_ids": [W, P, P, P, i32, i32, P, P, P],
            "xpress_jacobi_step": [W, P, P, i64, P, P, i32, i32, i32, ctypes.c_uint32, P, P, P,
                                   sz, P],
            "xpress_jacobi_step_noalloc": [W, P, P, i64, P, P, i32, i32, i32, ctypes.c_uint32,
                                           P, P, P],
            "xpress_jacobi_step_graph": [W, P, P, i64, P, P, i32, i32, i32, ctypes.c_uint32, P, P,
                                         P, sz, ctypes.POINTER(ctypes.c_void_p)],
            "xpress_graph_launch": [P, P],
            "xpress_graph_destroy": [P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.xpress_last_error.restype = ctypes.c_char_p
        L.xpress_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != OK:
        msg = lib().xpress_last_error().decode()
        raise XpressError(status, msg)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _bf16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA bfloat16 tensor")
    return t


def _at_least(t, n: int, name: str) -> None:
    """The C ABI takes bare pointers and a block count: a tensor shorter than that count implies
    would be read or written past its end, so it is refused here."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, fewer than the {n} that N implies")


def _base_rows(base, rows: int, V: int) -> None:
    _bf16(base, "base")
    if base.stride(1) != 1 or base.dim() != 2:
        raise ValueError("base must be a [rows, V] view with unit column stride")
    if base.shape[0] < rows or base.shape[1] != V:
        raise ValueError(f"base is {tuple(base.shape)}; the call needs [{rows}, {V}]")


def _step_inputs(w, h, base, anchor, am1, blk) -> int:
    """N from blk [N, B]; h, base, anchor and am1 must cover N blocks."""
    d = w.dims
    N, B = blk.shape
    if B != d["B"]:
        raise ValueError(f"blk has {B} slots per block, the weights {d['B']}")
    _at_least(_bf16(h, "h"), N * B * d["H"], "h")
    _base_rows(base, N * (B - 1), d["V"])
    _at_least(anchor, N, "anchor")
    _at_least(am1, N, "am1")
    return N


@dataclass
class Weights:
    """Device bf16 weights of one refiner head, ``nn.Linear`` layouts; ``mix_L`` is folded and
    stored [B, B, r]."""

    w1: torch.Tensor
    down_h: torch.Tensor
    down_g: torch.Tensor
    in_proj: torch.Tensor
    mix_L: torch.Tensor
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    w2: torch.Tensor
    # optional fp32 [V, r] projected embedding table (fold_embedding); None: not used
    w1p: torch.Tensor | None = None

    @property
    def dims(self):
        V, r = self.w1.shape
        return dict(B=self.mix_L.shape[1], r=r, H=self.down_h.shape[1], M=self.w_gate.shape[0],
                    V=V)

    def struct(self) -> _Weights:
        d = self.dims
        s = _Weights(B=d["B"], r=d["r"], H=d["H"], M=d["M"], V=d["V"])
        for k in ("w1", "down_h", "down_g", "in_proj", "mix_L", "w_gate", "w_up", "w_down", "w2"):
            t = _bf16(getattr(self, k), k)
            if not t.is_contiguous():
                raise ValueError(f"{k} must be contiguous")
            setattr(s, k, t.data_ptr())
        if self.w1p is not None:
            t = self.w1p
            if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
                raise TypeError("w1p must be a contiguous CUDA float32 tensor")
            if tuple(t.shape) != (d["V"], d["r"]):
                raise ValueError(f"w1p shape {tuple(t.shape)} != (V, r) = ({d['V']}, {d['r']})")
            s.w1p = t.data_ptr()
        return s


def workspace_size(n_max: int, B: int, r: int, V: int, C: int, k_max: int) -> int:
    out = ctypes.c_size_t()
    _check(lib().xpress_workspace_size(n_max, B, r, V, C, k_max, ctypes.byref(out)))
    return int(out.value)


def alloc_workspace(n_max: int, B: int, r: int, V: int, C: int, k_max: int, device="cuda"):
    n = workspace_size(n_max, B, r, V, C, k_max)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def fold_mixer(raw: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """raw: [r, B, B] bf16 -> folded mixer [B, B, r] (channel innermost)."""
    raw = _bf16(raw, "raw").contiguous()
    r, B, _ = raw.shape
    out = torch.empty(B, B, r, dtype=raw.dtype, device=raw.device) if out is None else out
    _check(lib().xpress_fold_mixer(_ptr(raw), r, B, _ptr(out), _stream()))
    return out


def fold_embedding(w: Weights, out: torch.Tensor | None = None) -> torch.Tensor:
    """Projected embedding table w1p [V, r] fp32: in_proj's embedding block applied to every row
    of w1 (set it as ``w.w1p`` to run the latent stage as two launches instead of three)."""
    d = w.dims
    s = w.struct()
    out = (torch.empty(d["V"], d["r"], dtype=torch.float32, device=w.w1.device)
           if out is None else out)
    _check(lib().xpress_fold_embedding(ctypes.byref(s), _ptr(out), _stream()))
    return out


def hidden_cache(w: Weights, h: torch.Tensor, xh: torch.Tensor, ws: torch.Tensor) -> torch.Tensor:
    s = w.struct()
    N = h.shape[0]
    _at_least(_bf16(h, "h"), N * w.dims["B"] * w.dims["H"], "h")
    _at_least(xh, N * w.dims["B"] * w.dims["r"], "xh")
    _check(lib().xpress_hidden_cache(ctypes.byref(s), _ptr(_bf16(h, "h")), N, _ptr(xh), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream()))
    return xh


def initial_block(base: torch.Tensor, anchor: torch.Tensor, blk: torch.Tensor) -> torch.Tensor:
    N, B = blk.shape
    _base_rows(base, N * (B - 1), base.shape[1])
    _at_least(anchor, N, "anchor")
    _check(lib().xpress_initial_block(ctypes.c_void_p(base.data_ptr()), base.stride(0),
                                      _ptr(anchor), N, B, base.shape[1], _ptr(blk), _stream()))
    return blk


def lat_buffer(N: int, B: int, r: int, layout: int = LAT_ROWS, device="cuda") -> torch.Tensor:
    """A latent buffer for N blocks in `layout` (fragment order: whole 32-row tiles)."""
    rows = N * (B - 1)
    if layout == LAT_FRAGMENTS:
        rows = (rows + 31) // 32 * 32
    return torch.empty(rows, r, dtype=torch.bfloat16, device=device)


def latent_pass(w: Weights, blk, am1, xh, lat, ws: torch.Tensor, layout: int = LAT_ROWS) -> torch.Tensor:
    s = w.struct()
    N = blk.shape[0]
    _at_least(am1, N, "am1")
    _at_least(xh, N * w.dims["B"] * w.dims["r"], "xh")
    _at_least(lat, N * (w.dims["B"] - 1) * w.dims["r"], "lat")
    _check(lib().xpress_latent_pass(ctypes.byref(s), _ptr(blk), _ptr(am1), _ptr(xh), N,
                                    _ptr(lat), layout, _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream()))
    return lat


def readout_argmax(w: Weights, lat, base, blk, ws, changed=None, layout: int = LAT_ROWS) -> torch.Tensor:
    s = w.struct()
    N = blk.shape[0]
    _base_rows(base, N * (w.dims["B"] - 1), w.dims["V"])
    _at_least(lat, N * (w.dims["B"] - 1) * w.dims["r"], "lat")
    _check(lib().xpress_readout_argmax(ctypes.byref(s), _ptr(lat), layout,
                                       ctypes.c_void_p(base.data_ptr()), base.stride(0), N,
                                       _ptr(blk), _ptr(changed), _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream()))
    return blk


def readout_tiles(V: int, rows: int) -> int:
    out = ctypes.c_int32()
    _check(lib().xpress_readout_tiles(V, rows, ctypes.byref(out)))
    return int(out.value)


def readout_partials(w: Weights, lat, base, part: torch.Tensor, layout: int = LAT_ROWS) -> torch.Tensor:
    """part: int32/uint32-compatible tensor [ntiles, rows, 2] (value bits, id), range-major."""
    s = w.struct()
    rows = part.shape[1]
    N = rows // (w.dims["B"] - 1)
    _base_rows(base, N * (w.dims["B"] - 1), w.dims["V"])
    _at_least(lat, N * (w.dims["B"] - 1) * w.dims["r"], "lat")
    _check(lib().xpress_readout_partials(ctypes.byref(s), _ptr(lat), layout,
                                         ctypes.c_void_p(base.data_ptr()), base.stride(0), N,
                                         _ptr(part), _stream()))
    return part


def argmax_reduce(part: torch.Tensor, blk: torch.Tensor, changed=None) -> torch.Tensor:
    N, B = blk.shape
    ntiles = part.shape[0]
    _check(lib().xpress_argmax_reduce(_ptr(part), ntiles, N, B, _ptr(blk), _ptr(changed),
                                      _stream()))
    return blk


def topc_prepare(w: Weights, base, N: int, C: int, cand, base_c, w2c=None, ws=None):
    """w2c None: candidates and base_c only (for readout_argmax_topc_ids)."""
    s = w.struct()
    _base_rows(base, N * (w.dims["B"] - 1), w.dims["V"])
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().xpress_topc_prepare(ctypes.byref(s), ctypes.c_void_p(base.data_ptr()),
                                     base.stride(0), N, C, _ptr(cand), _ptr(base_c), _ptr(w2c),
                                     _ptr(ws), nbytes, _stream()))
    return cand, base_c, w2c


def readout_argmax_topc(lat, w2c, base_c, cand, blk, changed=None) -> torch.Tensor:
    N, B = blk.shape
    rows, c, r = w2c.shape
    _check(lib().xpress_readout_argmax_topc(_ptr(lat), _ptr(w2c), _ptr(base_c), _ptr(cand), N, B,
                                            r, c, _ptr(blk), _ptr(changed), _stream()))
    return blk


def readout_argmax_topc_ids(w: Weights, lat, base_c, cand, blk, changed=None) -> torch.Tensor:
    """The top-C readout reading w2[cand] through the ids (no gathered copy)."""
    s = w.struct()
    N = blk.shape[0]
    c = cand.shape[-1]
    _check(lib().xpress_readout_argmax_topc_ids(ctypes.byref(s), _ptr(lat), _ptr(base_c),
                                                _ptr(cand), N, c, _ptr(blk), _ptr(changed),
                                                _stream()))
    return blk


def jacobi_step(w: Weights, h, base, anchor, am1, blk, *, K: int, C: int = 0,
                flags: int = INIT_FROM_BASE, ws: torch.Tensor, passes_run=None) -> torch.Tensor:
    s = w.struct()
    N = _step_inputs(w, h, base, anchor, am1, blk)
    _check(lib().xpress_jacobi_step(ctypes.byref(s), _ptr(_bf16(h, "h")),
                                    ctypes.c_void_p(base.data_ptr()), base.stride(0), _ptr(anchor),
                                    _ptr(am1), N, K, C, flags, _ptr(blk), _ptr(passes_run),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return blk


def jacobi_step_noalloc(w: Weights, h, base, anchor, am1, blk, *, K: int, C: int = 0,
                        flags: int = INIT_FROM_BASE, passes_run=None) -> torch.Tensor:
    """``jacobi_step`` on the library's own static per-GPU scratch: no workspace argument and no
    allocation. Calls that overlap on one GPU share that scratch and race."""
    s = w.struct()
    N = _step_inputs(w, h, base, anchor, am1, blk)
    _check(lib().xpress_jacobi_step_noalloc(ctypes.byref(s), _ptr(_bf16(h, "h")),
                                            ctypes.c_void_p(base.data_ptr()), base.stride(0),
                                            _ptr(anchor), _ptr(am1), N, K, C, flags, _ptr(blk),
                                            _ptr(passes_run), _stream()))
    return blk


class StepGraph:
    """A draft step recorded once as a HIP graph (``xpress_jacobi_step_graph``); ``launch()``
    replays the whole step on the current stream with one call. The tensors given at creation are
    kept referenced: the graph reads and writes them in place on every launch."""

    def __init__(self, w: Weights, h, base, anchor, am1, blk, *, K: int, C: int = 0,
                 flags: int = INIT_FROM_BASE, ws: torch.Tensor, passes_run=None):
        s = w.struct()
        N = _step_inputs(w, h, base, anchor, am1, blk)
        self._keep = (w, h, base, anchor, am1, blk, ws, passes_run)
        self._handle = ctypes.c_void_p()
        _check(lib().xpress_jacobi_step_graph(
            ctypes.byref(s), _ptr(_bf16(h, "h")), ctypes.c_void_p(base.data_ptr()),
            base.stride(0), _ptr(anchor), _ptr(am1), N, K, C, flags, _ptr(blk), _ptr(passes_run),
            _ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(self._handle)))

    def launch(self) -> None:
        if not self._handle:
            raise RuntimeError("graph was closed")
        _check(lib().xpress_graph_launch(self._handle, _stream()))

    def close(self) -> None:
        if self._handle:
            _check(lib().xpress_graph_destroy(self._handle))
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
