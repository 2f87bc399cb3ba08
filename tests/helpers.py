"""Shared helpers for the tests (no computation of the method lives here)."""

import numpy as np
import torch

# Tolerances of the GPU path against the fp64 oracle on unit-scale inputs.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5
# lse of the bf16 varlen kernel is the log of the row sum of the softmax
# weights after their rounding to bf16 (the same weights that multiply V, so
# the output's weights sum to one).  Round-to-nearest to bf16's 8-bit
# significand changes each weight by a relative 2^-8 at most, so the row sum,
# and with it exp(lse), by the same: |d lse| <= ln(1 + 2^-8) = 3.9e-3, plus
# fp32 accumulation error far below that.  The roundings are unbiased: over
# rows that hold a single weight (the worst case, no averaging) the mean of
# |d lse| is 1.41e-3 for weights spread over an octave, so a systematic
# offset of 2e-3 fails the mean bound.  The fp32 path sums unrounded weights.
LSE_ATOL_BF16 = 4e-3
LSE_MEAN_BF16 = 2e-3
LSE_ATOL_F32 = 1e-5


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(got: np.ndarray, ref: np.ndarray, f32: bool, what: str):
    err = np.abs(got - ref)
    if f32:
        assert err.max() <= F32_MAX_ABS, f"{what}: max-abs {err.max():.3g} > {F32_MAX_ABS}"
    else:
        assert err.max() <= BF16_MAX_ABS, f"{what}: max-abs {err.max():.3g} > {BF16_MAX_ABS}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean-abs {err.mean():.3g} > {BF16_MEAN_ABS}"
    return float(err.max()), float(err.mean())


def check_lse(got: np.ndarray, ref: np.ndarray, f32: bool, what: str):
    both_inf = np.isneginf(got) & np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    d = np.abs(got[~both_inf] - ref[~both_inf])
    tol = LSE_ATOL_F32 if f32 else LSE_ATOL_BF16
    if d.size:
        print(f"[lse] {what}: max-abs {d.max():.3g} mean-abs {d.mean():.3g}", flush=True)
        assert d.max() <= tol, f"{what}: lse max-abs {d.max():.3g} > {tol}"
        if not f32:
            assert d.mean() <= LSE_MEAN_BF16, f"{what}: lse mean-abs {d.mean():.3g} > {LSE_MEAN_BF16}"


def sample_rows(cu, block_m: int = 128, n_random: int = 256, seed: int = 0, edge: int = 64):
    """Rows to compare on large inputs: each request's first and last `edge`
    rows, rows on both sides of every q-tile boundary, and random rows."""
    cu = [int(x) for x in cu]
    rows = set()
    for r in range(len(cu) - 1):
        a, b = cu[r], cu[r + 1]
        rows.update(range(a, min(b, a + edge)))
        rows.update(range(max(a, b - edge), b))
        for t in range(a + block_m, b, block_m):
            rows.update((t - 1, t))
    rng = np.random.default_rng(seed)
    if cu[-1] > 0:
        rows.update(int(x) for x in rng.integers(0, cu[-1], size=n_random))
    return np.array(sorted(rows), dtype=np.int64)
