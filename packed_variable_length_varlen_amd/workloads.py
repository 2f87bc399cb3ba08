"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
attention, packing or boundary arithmetic.  Both the GPU path and the CPU
oracle are fed from what it returns.

Recipe (all workloads):
  * rng = numpy.random.default_rng(seed), seed = the spec's seed field;
  * per-request text lengths are drawn first, in request order, with
    rng.integers(lo, hi + 1);
  * then Q, K and V are drawn in that order, each as float32 standard normals,
    request by request, text piece then image piece;
  * bf16 tensors are the float32 draws rounded once to bfloat16 (round to
    nearest even).

The shapes follow the pages' workloads: a 2048x2048 image is a 128x128 grid of
16,384 tokens and a 1328x1328 image an 83x83 grid of 6,889 tokens (PR #4293
discussion of sequence lengths); text is at most 256 tokens in a padded text
buffer; the vocoder DiT uses 24-frame blocks (PR #7975).  The real prompts,
images and audio of the pages are not used: N(0, 1) tensors of those shapes
stand in for them.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np
import torch

TEXT_CAP = 256  # width of the padded per-request text buffer


@dataclass
class VarlenSpec:
    """A packed joint text+image batch: per request (text length range, grid)."""
    name: str
    H: int
    D: int
    text_ranges: List[Tuple[int, int]]        # inclusive (lo, hi) per request; lo == hi for fixed
    img_grids: List[Tuple[int, int]]          # (h, w) per request; (0, 0) = no image part
    seed: int


@dataclass
class BlockLocalSpec:
    name: str
    B: int
    n: int
    H: int
    D: int
    block: int
    windows: List[Tuple[int, int]]            # (look_back, look_ahead) per call
    seed: int


WORKLOADS = {
    # 3 packed requests of 17, 64 and 129 tokens (text-only pieces), H=2, D=64.
    "tiny-3req": VarlenSpec("tiny-3req-17-64-129-h2-d64", 2, 64,
                  [(17, 17), (64, 64), (129, 129)], [(0, 0), (0, 0), (0, 0)], 1),
    # One joint request: 2048x2048 image -> 128x128 grid, text 8..256.
    "joint-16k": VarlenSpec("joint-1req-2048sq-16384img-text8-256-h24-d128", 24, 128,
                  [(8, 256)], [(128, 128)], 2),
    # Mixed resolutions: 64x64, 83x83, 128x128, 48x84 grids, each after text 8..256.
    "mixres-4req": VarlenSpec("mixres-4req-4096-6889-16384-4032img-h24-d128", 24, 128,
                  [(8, 256)] * 4, [(64, 64), (83, 83), (128, 128), (48, 84)], 3),
    # Edit-style CFG halves [r1+, r1-, r2+, r2-]: 2x16,384 image tokens each
    # (noise + source latents, a 256x128 grid), positive text 8..256,
    # negative text 1..8.
    "edit-cfg-4seq": VarlenSpec("edit-cfg-4seq-32768img-h24-d128", 24, 128,
                  [(8, 256), (1, 8), (8, 256), (1, 8)], [(256, 128)] * 4, 4),
}

BLOCK_LOCAL_WORKLOADS = {
    "vocoder-dit": BlockLocalSpec("dit-blocklocal-n2003-b24-h16-d64", 1, 2003, 16, 64, 24,
                      [(0, 0), (1, 0), (0, 1), (1, 1)], 5),
}


@dataclass
class VarlenInputs:
    spec: VarlenSpec
    dtype: torch.dtype
    text_len: List[int]
    img_hw: List[Tuple[int, int]]
    text_mask: np.ndarray                      # bool [R, TEXT_CAP]
    img_tokens: List[int]                      # h*w per request (sizes of the drawn pieces)
    img_cap: int                               # slab width of the padded image buffers
    q_text: torch.Tensor                       # [R, TEXT_CAP, H, D], zero in the padding
    k_text: torch.Tensor
    v_text: torch.Tensor
    q_img: torch.Tensor                        # [R, img_cap, H, D], zero in the padding
    k_img: torch.Tensor
    v_img: torch.Tensor
    scale: float                               # float32(1/sqrt(D)) as a Python float

    @property
    def R(self) -> int:
        return len(self.text_len)

    @property
    def total_tokens(self) -> int:
        return sum(self.text_len) + sum(self.img_tokens)

    @property
    def max_len(self) -> int:
        return max(t + n for t, n in zip(self.text_len, self.img_tokens))


def _to(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def softmax_scale(D: int) -> float:
    """1/sqrt(D) rounded to float32, returned as a Python float."""
    return float(np.float32(1.0 / np.sqrt(np.float64(D))))


def make_varlen_inputs(spec: VarlenSpec, dtype: torch.dtype = torch.bfloat16,
                       seed: Optional[int] = None) -> VarlenInputs:
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    R = len(spec.text_ranges)
    text_len = [int(rng.integers(lo, hi + 1)) for lo, hi in spec.text_ranges]
    img_tokens = [int(h) * int(w) for h, w in spec.img_grids]
    img_cap = max(img_tokens) if img_tokens else 0
    H, D = spec.H, spec.D
    text_mask = np.zeros((R, TEXT_CAP), dtype=bool)
    for r, t in enumerate(text_len):
        text_mask[r, :t] = True
    slabs = {}
    for name in ("q", "k", "v"):
        tb = np.zeros((R, TEXT_CAP, H, D), dtype=np.float32)
        ib = np.zeros((R, img_cap, H, D), dtype=np.float32)
        for r in range(R):
            tb[r, :text_len[r]] = rng.standard_normal((text_len[r], H, D), dtype=np.float32)
            ib[r, :img_tokens[r]] = rng.standard_normal((img_tokens[r], H, D), dtype=np.float32)
        slabs[name] = (_to(tb, dtype), _to(ib, dtype))
    return VarlenInputs(spec, dtype, text_len, list(spec.img_grids), text_mask, img_tokens, img_cap,
                        slabs["q"][0], slabs["k"][0], slabs["v"][0],
                        slabs["q"][1], slabs["k"][1], slabs["v"][1], softmax_scale(D))


def varlen_lengths(spec: VarlenSpec, seed: Optional[int] = None) -> List[int]:
    """Per-request joint lengths (text + image tokens) of a workload: the text
    lengths are the same first draws of the same generator as in
    make_varlen_inputs, without drawing the tensors."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    text_len = [int(rng.integers(lo, hi + 1)) for lo, hi in spec.text_ranges]
    return [t + int(h) * int(w) for t, (h, w) in zip(text_len, spec.img_grids)]


def random_varlen_case(seed: int, lengths: List[int], H: int, D: int, dtype: torch.dtype,
                       kv_lengths: Optional[List[int]] = None):
    """Packed q [sum(lengths), H, D] and k/v [sum(kv_lengths), H, D] N(0,1) draws
    for small ad-hoc cases (edge cases: empty requests, q != kv lengths)."""
    rng = np.random.default_rng(seed)
    kv_lengths = lengths if kv_lengths is None else kv_lengths
    q = rng.standard_normal((sum(lengths), H, D), dtype=np.float32)
    k = rng.standard_normal((sum(kv_lengths), H, D), dtype=np.float32)
    v = rng.standard_normal((sum(kv_lengths), H, D), dtype=np.float32)
    return _to(q, dtype), _to(k, dtype), _to(v, dtype)


@dataclass
class BlockLocalInputs:
    spec: BlockLocalSpec
    dtype: torch.dtype
    q: torch.Tensor                            # [B, n, H, D]
    k: torch.Tensor
    v: torch.Tensor
    scale: float


def make_block_local_inputs(spec: BlockLocalSpec, dtype: torch.dtype = torch.bfloat16,
                            seed: Optional[int] = None, n: Optional[int] = None,
                            B: Optional[int] = None) -> BlockLocalInputs:
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    n = spec.n if n is None else n
    B = spec.B if B is None else B
    shape = (B, n, spec.H, spec.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return BlockLocalInputs(spec, dtype, _to(q, dtype), _to(k, dtype), _to(v, dtype), softmax_scale(spec.D))
