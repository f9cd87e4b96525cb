"""Seeded synthetic inputs for the XPress Jacobi refinement pass.

This module only draws data. It holds none of the method's arithmetic: no fold of the mixer, no
projection, no readout, no argmax of anything the method computes. Both the CPU oracle (under
``oracle/``) and the HIP path take their inputs from here, so neither side ever supplies the
other's inputs.

Every workload is drawn with NumPy's PCG64 generator (``numpy.random.default_rng(seed)``) in the
order the fields are listed in ``_DRAW_ORDER``. Normal draws are made in float64 by NumPy, cast to
float32, and, for the bfloat16 workloads, rounded to bfloat16 with round-to-nearest-even. Values are
always handed out as float32 arrays that hold exactly the bf16 (or fp32) values; ``bf16_bits`` gives
the 16-bit patterns the device buffers hold.

The workloads are the five sizes the method is measured on: a tiny fp32 case that the oracle runs
to the fixed point, a single request, a 32-block batch (full vocabulary and top-C) and a 256-block
batch. Shapes follow the parameter set of ``XPressRefinerHead`` (qwen3_xpress API page, constructor)
in the ``nn.Linear`` layouts ``[out_features, in_features]``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

__all__ = [
    "WORKLOADS",
    "Workload",
    "Inputs",
    "bf16_round",
    "bf16_bits",
    "bits_to_f32",
    "make_inputs",
]


@dataclass(frozen=True)
class Workload:
    """Sizes and value recipe of one synthetic workload."""

    name: str
    N: int  # blocks (requests)
    B: int  # slots per block; slot 0 is the verified anchor
    r: int  # latent rank
    H: int  # model hidden size
    M: int  # SwiGLU hidden size (mlp_hidden)
    V: int  # vocabulary size
    C: int  # top-C candidates per row; 0 scores the full vocabulary
    K: int  # Jacobi passes per step (0: run to the fixed point, at most B-1 passes + 1 check)
    bf16: bool  # weights and inputs are bf16 values (False: fp32 draws)
    w_std: float = 0.02
    mix_std: float = 0.05
    base_std: float = 2.0
    boost: float = 0.0  # added to one uniformly drawn token per base row
    dup_frac: float = 0.0  # fraction of base rows whose maximum is copied to a second token

    @property
    def rows(self) -> int:
        return self.N * (self.B - 1)


WORKLOADS: dict[int, Workload] = {
    1: Workload("tiny_fp32_fixed_point", N=2, B=4, r=64, H=256, M=128, V=8192, C=0, K=0,
                bf16=False, w_std=0.02, mix_std=0.1, base_std=1.0),
    2: Workload("single_request_full_vocab", N=1, B=16, r=256, H=4096, M=512, V=151936, C=0,
                K=15, bf16=True, boost=6.0),
    3: Workload("batch32_full_vocab", N=32, B=16, r=256, H=4096, M=512, V=151936, C=0, K=15,
                bf16=True, boost=6.0),
    4: Workload("batch32_top512", N=32, B=16, r=256, H=5120, M=512, V=151936, C=512, K=15,
                bf16=True, boost=6.0),
    5: Workload("batch256_full_vocab_dupmax", N=256, B=16, r=256, H=5120, M=512, V=151936, C=0,
                K=15, bf16=True, dup_frac=0.2),
}

# Draw order (fixes which random numbers land where for a given seed).
_DRAW_ORDER = ("w1", "down_h", "down_g", "in_proj", "w_gate", "w_up", "w_down", "w2",
               "raw_L", "h", "base", "blk", "am1")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 patterns of float32 ``x``, rounded to nearest, ties to even.

    Inputs are finite by construction; NaN/Inf handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """float32 values of uint16 bfloat16 patterns (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array holding ``x`` rounded to the nearest bfloat16 value (ties to even)."""
    return bits_to_f32(bf16_bits(x))


@dataclass
class Inputs:
    """One draw of every tensor a step consumes. Float fields are float32 arrays.

    ``base`` holds the base logits of the draft slots only, ``[N*(B-1), V]``; row
    ``n*(B-1) + b-1`` belongs to slot ``b`` of block ``n``. ``blk[:, 0]`` is the verified anchor.
    """

    wl: Workload
    w1: np.ndarray  # [V, r] token embedding
    down_h: np.ndarray  # [r, H]
    down_g: np.ndarray  # [r, H]
    in_proj: np.ndarray  # [r, 3r]
    w_gate: np.ndarray  # [M, r]
    w_up: np.ndarray  # [M, r]
    w_down: np.ndarray  # [r, M]
    w2: np.ndarray  # [V, r] readout
    raw_L: np.ndarray  # [r, B, B] raw (unfolded) per-channel mixer
    h: np.ndarray  # [N, B, H] hidden states
    base: np.ndarray  # [N*(B-1), V] base logits of the draft slots
    blk: np.ndarray  # [N, B] int64 starting block; column 0 is the anchor
    am1: np.ndarray  # [N] int64 token before each anchor
    meta: dict = field(default_factory=dict)

    FLOAT_FIELDS = ("w1", "down_h", "down_g", "in_proj", "w_gate", "w_up", "w_down", "w2",
                    "raw_L", "h", "base")

    @property
    def anchor(self) -> np.ndarray:
        return self.blk[:, 0].copy()

    def rounded_bf16(self) -> "Inputs":
        """A copy whose float tensors are rounded to bf16 (what a bf16 device buffer holds)."""
        if self.wl.bf16:
            return self
        return replace(self, **{k: bf16_round(getattr(self, k)) for k in self.FLOAT_FIELDS})


def _normal(rng: np.random.Generator, shape, std: float, chunk: int = 1 << 24) -> np.ndarray:
    """float32 N(0, std^2) draws, produced in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s) * std
    return out.reshape(shape)


def make_inputs(wl: Workload | int, seed: int = 0, *, N: int | None = None) -> Inputs:
    """Draw one workload. ``N`` overrides the block count (for small parity cases)."""
    if isinstance(wl, int):
        wl = WORKLOADS[wl]
    if N is not None:
        wl = replace(wl, N=N)
    rng = np.random.default_rng(seed)
    rnd = bf16_round if wl.bf16 else (lambda a: a)
    N_, B, r, H, M, V = wl.N, wl.B, wl.r, wl.H, wl.M, wl.V
    rows = N_ * (B - 1)
    meta: dict = {"seed": seed}
    d: dict[str, np.ndarray] = {}
    shapes = {
        "w1": (V, r), "down_h": (r, H), "down_g": (r, H), "in_proj": (r, 3 * r),
        "w_gate": (M, r), "w_up": (M, r), "w_down": (r, M), "w2": (V, r),
    }
    for name in _DRAW_ORDER:
        if name in shapes:
            d[name] = rnd(_normal(rng, shapes[name], wl.w_std))
        elif name == "raw_L":
            d[name] = rnd(_normal(rng, (r, B, B), wl.mix_std))
        elif name == "h":
            d[name] = rnd(_normal(rng, (N_, B, H), 1.0))
        elif name == "base":
            base = _normal(rng, (rows, V), wl.base_std)
            if wl.boost:
                ids = rng.integers(0, V, size=rows)
                base[np.arange(rows), ids] += np.float32(wl.boost)
                meta["boost_ids"] = ids
            base = rnd(base)
            if wl.dup_frac:
                # Copy each chosen row's largest value to a second, uniformly drawn token, so the
                # row's maximum occurs (at least) twice.
                pick = rng.random(rows) < wl.dup_frac
                second = rng.integers(0, V, size=rows)
                sel = np.nonzero(pick)[0]
                top = base[sel].max(axis=1)
                base[sel, second[sel]] = top
                meta["dup_rows"] = sel
                meta["dup_ids"] = second[sel]
            d[name] = base
        elif name == "blk":
            d[name] = rng.integers(0, V, size=(N_, B), dtype=np.int64)
        elif name == "am1":
            d[name] = rng.integers(0, V, size=(N_,), dtype=np.int64)
    return Inputs(wl=wl, meta=meta, **d)
