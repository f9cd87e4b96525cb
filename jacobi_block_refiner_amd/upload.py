"""Upload of host inputs (NumPy float32 arrays) to device bf16 tensors for the C ABI.

Marshalling only: values are rounded to bf16 (round to nearest even) on the host, the raw mixer is
folded into its serving form by the library's own ``xpress_fold_mixer``, and the projected
embedding table is built by ``xpress_fold_embedding``.
"""
from __future__ import annotations

import numpy as np
import torch

from . import synth, xpress


def bf16_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    bits = synth.bf16_bits(np.asarray(a, dtype=np.float32))
    return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)


def weights(inp: synth.Inputs, device="cuda", *, embed_table: bool = True) -> xpress.Weights:
    """Device weights; with ``embed_table`` also the projected embedding table (built by the
    library's ``xpress_fold_embedding``), which runs the latent stage as two launches instead of three."""
    raw = bf16_tensor(inp.raw_L, device)
    w = xpress.Weights(
        w1=bf16_tensor(inp.w1, device), down_h=bf16_tensor(inp.down_h, device),
        down_g=bf16_tensor(inp.down_g, device), in_proj=bf16_tensor(inp.in_proj, device),
        mix_L=xpress.fold_mixer(raw), w_gate=bf16_tensor(inp.w_gate, device),
        w_up=bf16_tensor(inp.w_up, device), w_down=bf16_tensor(inp.w_down, device),
        w2=bf16_tensor(inp.w2, device))
    if embed_table:
        w.w1p = xpress.fold_embedding(w)
    return w


def base_logits(base: np.ndarray, device="cuda") -> torch.Tensor:
    """[rows, V] bf16 view whose row stride is V rounded up to a multiple of 8."""
    rows, V = base.shape
    ld = (V + 7) // 8 * 8
    if ld == V:
        return bf16_tensor(base, device)
    buf = torch.zeros(rows, ld, dtype=torch.bfloat16, device=device)
    buf[:, :V] = bf16_tensor(base, device)
    return buf[:, :V]


def tokens(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(device)
