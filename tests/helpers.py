"""Shared helpers for the tests (no computation of the method lives here)."""

import numpy as np
import torch

# Tolerances of the GPU path against the fp64 oracle on unit-scale inputs.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-5
# lse tolerances (the pages define no lse; these follow from the arithmetic).
# The bf16 varlen kernels normalise by the row sum of the softmax weights
# after their rounding to bf16 (the same weights that multiply V, so the
# output's weights sum to one).  Max bound: round-to-nearest to bf16's 8-bit
# significand moves a weight x in [2^e, 2^(e+1)) by at most 2^(e-8), a
# relative 2^-8, so the row sum -- hence exp(lse) -- moves by at most that
# relative amount: |d lse| <= -ln(1 - 2^-8) = 3.9e-3 (fp32 accumulation adds
# orders of magnitude less).  Mean bound: the rounding error of x is uniform
# on [-2^(e-8), 2^(e-8)], mean |error| 2^(e-9); the kernel's exponent offset
# is an integer, so a row's largest weight is 2^f with f the fractional part
# of its scaled maximum score, uniform on (-1, 0] for these random inputs.
# For a row whose sum is one weight (no averaging: the worst case) the mean
# relative error is 2^-9 * E[2^-t], t uniform on [0, 1), = 2^-9 * (1/2) / ln 2
# = 1.41e-3; rows with several comparable weights average their independent
# roundings and lie below that.  The test bound is 2e-3, the 1.41e-3
# expectation plus room for the sampling spread of a case's mean.
# Kernels that sum the unrounded fp32 weights (the fp32 paths and every
# block-local kernel, bf16 included) carry only fp32 error: scores of
# unit-scale inputs are exact products summed in fp32, exp2/log2 are within a
# few ulps, so |d lse| stays near 1e-6 and is tested at 1e-5.
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


def check_lse(got: np.ndarray, ref: np.ndarray, f32: bool, what: str, rounded_weights: bool = True):
    """lse against the oracle.  rounded_weights: the kernel sums the bf16-rounded
    weights (the bf16 varlen kernels); False for kernels that sum fp32 weights."""
    both_inf = np.isneginf(got) & np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{what}: -inf pattern differs"
    d = np.abs(got[~both_inf] - ref[~both_inf])
    rounded = rounded_weights and not f32
    tol = LSE_ATOL_BF16 if rounded else LSE_ATOL_F32
    if d.size:
        print(f"[lse] {what}: max-abs {d.max():.3g} mean-abs {d.mean():.3g}", flush=True)
        assert d.max() <= tol, f"{what}: lse max-abs {d.max():.3g} > {tol}"
        if rounded:
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
