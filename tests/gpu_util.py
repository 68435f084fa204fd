"""Helpers shared by the GPU parity tests (not collected by pytest).

Tolerances (from the method's numeric contract: bf16 in, fp32 accumulate):
attention outputs max-abs <= 1e-2 (plus, for outputs stored in bf16, the
bf16 rounding of the value itself) and mean-abs <= 1e-3, log-sum-exp values
|d| <= 1e-3, and no NaN/Inf anywhere.
"""
import math

import numpy as np
import torch

from oracle.star_oracle import round_bf16
from workloads import bf16_bits_to_f32, draw_tensor

OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def to_dev(x: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor; float32 -> fp32."""
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def rand_tensor(seed, tid, B, H, S, D, scale=1.0, bf16=True):
    return draw_tensor(seed, tid, B, H, S, D, scale, as_bf16=bf16)


def check_out(got: np.ndarray, ref: np.ndarray, what: str,
              max_abs=OUT_MAX_ABS, mean_abs=OUT_MEAN_ABS, bf16_out=False):
    """Element-wise max-abs and overall mean-abs bounds.  For a bf16 output
    (Phase-1 O, layer outputs) the bound on an element also admits the
    rounding of that output to bf16, at most 2^-8 |ref| (half an ulp,
    relative to the value): a stored bf16 value of magnitude above ~2.5
    cannot be within 1e-2 of the exact result; and the mean is taken
    against the exact result rounded to bf16."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    lim = max_abs + (2.0 ** -8) * np.abs(ref) if bf16_out else max_abs
    mx = float(err.max(initial=0.0))
    # the mean is taken against the exact value as the output dtype stores
    # it: rounding unit-scale values to bf16 alone costs ~1e-3 on average
    merr = np.abs(got - round_bf16(ref)) if bf16_out else err
    mn = float(merr.mean()) if merr.size else 0.0
    ok = bool((err <= lim).all())
    assert ok and mn <= mean_abs, f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}"
    return mx, mn


def check_lse(got: np.ndarray, ref: np.ndarray, what: str, tol=LSE_ABS):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert not np.isnan(got).any(), f"{what}: NaN"
    ninf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf_ref), f"{what}: -inf pattern differs"
    assert np.isfinite(got[~ninf_ref]).all(), f"{what}: non-finite lse"
    err = np.abs(got[~ninf_ref] - ref[~ninf_ref])
    mx = float(err.max(initial=0.0))
    assert mx <= tol, f"{what}: lse max-abs {mx:.3e}"
    return mx


def chunk_ranges(part_offsets, splits, align=64):
    """Chunk [start, end) ranges in o_part order, from the rule the header
    states: c_j = roundup(ceil(n_j / splits), align), chunk s of partition j
    is [off_j + s*c_j, min(off_j + (s+1)*c_j, off_{j+1}))."""
    out = []
    for j in range(len(part_offsets) - 1):
        a, b = part_offsets[j], part_offsets[j + 1]
        c = math.ceil((b - a) / splits)
        c = math.ceil(c / align) * align
        for s in range(splits):
            lo = a + s * c
            out.append((min(lo, b), max(min(lo + c, b), min(lo, b))))
    return out
