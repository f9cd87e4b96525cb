"""Shared pieces of the GPU parity tests: device upload, oracle runs on the same bf16 values, and
the agreement rules.

Agreement rules:
  * integer work (starting block, candidate sets, gathers, fold) is bit-exact;
  * readout tokens are bit-exact (lowest id on ties) except on rows whose oracle top-2 logit gap
    is below NEAR_TIE; on dyadic inputs, where every fp32 sum is exact, no row is exempt;
  * latents agree within LAT_RTOL of the row's largest magnitude (row-L-infinity relative).
"""
from __future__ import annotations

import sys
from dataclasses import replace

import numpy as np
import torch

from jacobi_block_refiner_amd import synth, upload, xpress
from oracle import oracle as O

NEAR_TIE = 1e-2
LAT_RTOL = 2e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def strong(inp):
    """Tiny workload (bf16 values) with weights scaled by powers of two so that tokens steer the
    readout and convergence takes several passes; scaling keeps every value bf16-exact."""
    b = inp.rounded_bf16()
    return replace(b, w1=b.w1 * 32, w2=b.w2 * 4, base=b.base * 0.25, in_proj=b.in_proj * 4,
                   w_gate=b.w_gate * 8, w_up=b.w_up * 8, w_down=b.w_down * 8)


def oracle_mixer(inp) -> np.ndarray:
    """The folded mixer as a bf16 parameter holds it (fold in double, then rounded to bf16)."""
    return synth.bf16_round(O.fold_mixer(inp.raw_L).astype(np.float32)).astype(np.float64)


class Dev:
    """Device copies of one workload's inputs."""

    def __init__(self, inp, device="cuda"):
        wl = inp.wl
        self.inp = inp
        self.w = upload.weights(inp, device)
        self.h = upload.bf16_tensor(inp.h, device)
        self.base = upload.base_logits(inp.base, device)
        self.am1 = upload.tokens(inp.am1, device)
        self.anchor = upload.tokens(inp.anchor, device)
        self.N, self.B, self.r, self.V = wl.N, wl.B, wl.r, wl.V
        self.rows = wl.N * (wl.B - 1)
        self.device = device

    def ws(self, C=0, K=16):
        return xpress.alloc_workspace(self.N, self.B, self.r, self.V, C, K, self.device)

    def xh(self):
        xh = torch.empty(self.N, self.B, self.r, dtype=torch.float32, device=self.device)
        xpress.hidden_cache(self.w, self.h, xh, self.ws())
        return xh

    def one_pass(self, blk_np, xh, ws=None, cand=None, base_c=None, w2c=None):
        """Latent + readout + argmax from the block blk_np; returns (new blk, lat)."""
        blk = upload.tokens(blk_np, self.device)
        lat = torch.empty(self.N, self.B - 1, self.r, dtype=torch.bfloat16, device=self.device)
        ws = ws if ws is not None else self.ws()
        xpress.latent_pass(self.w, blk, self.am1, xh, lat, ws)
        if cand is None:
            xpress.readout_argmax(self.w, lat, self.base, blk, ws if ws is not None else self.ws())
        else:
            xpress.readout_argmax_topc(lat, w2c, base_c, cand, blk)
        torch.cuda.synchronize()
        return blk.cpu().numpy(), lat


def lat_to_f64(lat: torch.Tensor) -> np.ndarray:
    return lat.float().cpu().numpy().astype(np.float64)


def lat_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """Largest over rows of max|got - want| / max|want| (row-L-infinity relative error)."""
    g = got.reshape(-1, got.shape[-1])
    w = want.reshape(-1, want.shape[-1])
    den = np.maximum(np.abs(w).max(axis=1), 1e-30)
    return float((np.abs(g - w).max(axis=1) / den).max())


def compare_tokens(got_rows: np.ndarray, want_rows: np.ndarray, gap: np.ndarray,
                   *, near_tie: float = NEAR_TIE):
    """Mismatches outside the near-tie exemption, and the exempt count."""
    exempt = gap < near_tie
    bad = (got_rows != want_rows) & ~exempt
    return int(bad.sum()), int(exempt.sum())


def draft_rows(blk: np.ndarray) -> np.ndarray:
    return blk[:, 1:].reshape(-1)


def end_to_end_ok(got: np.ndarray, want: np.ndarray, hist_gap: np.ndarray,
                  *, near_tie: float = NEAR_TIE):
    """End-to-end block agreement under the near-tie cascade rule: a mismatch at slot b of block n
    is allowed only if, in some pass, a row of that block at a slot b' <= b was a near tie
    (a legitimately different winner there changes every later slot's input). Returns
    (disallowed mismatches, exempt row-passes)."""
    N, B = got.shape
    near = (hist_gap < near_tie).reshape(hist_gap.shape[0], N, B - 1).any(axis=0)  # [N, B-1]
    allowed = np.zeros((N, B), bool)
    allowed[:, 1:] = np.logical_or.accumulate(near, axis=1)
    bad = (got != want) & ~allowed
    return int(bad.sum()), int((hist_gap < near_tie).sum())


def lat_pack_fragments(lat: np.ndarray) -> np.ndarray:
    """Row-major lat [rows, r] -> the readout's fragment order (XPRESS_LAT_FRAGMENTS), as a
    [ceil(rows/32)*32, r] array (rows past the end are zero): tile T, 16-channel group s, lane
    l = 32*h + i holds channels 16s + 8h .. +7 of row 32T + i. A pure permutation of the values."""
    rows, r = lat.shape
    nt = (rows + 31) // 32
    pad = np.zeros((nt * 32, r), dtype=lat.dtype)
    pad[:rows] = lat
    # [T, i, s, h, e] -> [T, s, h, i, e]
    return np.ascontiguousarray(pad.reshape(nt, 32, r // 16, 2, 8).transpose(0, 2, 3, 1, 4)).reshape(nt * 32, r)


def lat_unpack_fragments(frag: np.ndarray, rows: int) -> np.ndarray:
    """Inverse of lat_pack_fragments: the first `rows` rows, row-major."""
    n32, r = frag.shape
    nt = n32 // 32
    return np.ascontiguousarray(frag.reshape(nt, r // 16, 2, 32, 8).transpose(0, 3, 1, 2, 4)).reshape(nt * 32, r)[:rows]
