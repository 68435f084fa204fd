"""Helpers shared by the GPU parity tests (not collected by pytest).

Tolerances (from the method's numeric contract: bf16 in, fp32 accumulate):
attention outputs max-abs <= 1e-2 and mean-abs <= 1e-3 against the exact
result, log-sum-exp values |d| <= 1e-3, and no NaN/Inf anywhere.

An output stored in bf16 (Phase-1 O, layer outputs) may exceed 1e-2 only
where bf16 itself cannot do better: its element bound is
max(1e-2, 2^-8 |ref| + c), where 2^-8 |ref| is the value's own rounding to
bf16 (half an ulp) and c the compute error the kernel's arithmetic admits:
  * attention (``wabs`` given): c = 2^-9 wabs + 1e-4.  The kernel rounds each
    softmax weight to bf16 for the PV product (relative error 2^-9), which
    moves an output element by at most 2^-9 sum_i w_i |V_i,d| = 2^-9 wabs,
    the softmax average of |V| (the oracle's output for |V|); 1e-4 covers the
    fp32 accumulation.  For rows that see many keys c ~ 1e-3, so the bound is
    1e-2; it exceeds 1e-2 only in rows dominated by a few large values.
  * projections and layer outputs (``layer=True``), checked against the
    oracle fed the stage's actual bf16 input: c = LAYER_C = 1e-4, the fp32
    accumulation of a GEMM with K <= 4096 terms of unit-scale products.
The mean is taken against the exact result, except for the layer stages: a
unit-scale value rounded to bf16 alone is off by ~1.05e-3 on average, so
those are compared with the exact result rounded to bf16.
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


LAYER_C = 1e-4


def check_out(got: np.ndarray, ref: np.ndarray, what: str,
              max_abs=OUT_MAX_ABS, mean_abs=OUT_MEAN_ABS, bf16_out=False, wabs=None,
              layer=False):
    """Element-wise max-abs and overall mean-abs bounds (see the module
    docstring).  ``bf16_out``: the output is stored in bf16; then either
    ``wabs`` (the softmax average of |V| for every output element) or
    ``layer=True`` states the compute term."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    if bf16_out:
        if layer:
            c = LAYER_C
        else:
            assert wabs is not None and wabs.shape == ref.shape, f"{what}: wabs needed"
            c = 2.0 ** -9 * wabs + 1e-4
        lim = np.maximum(max_abs, (2.0 ** -8) * np.abs(ref) + c)
    else:
        lim = max_abs
    mx = float(err.max(initial=0.0))
    merr = np.abs(got - round_bf16(ref)) if (bf16_out and layer) else err
    mn = float(merr.mean()) if merr.size else 0.0
    bad = err > lim
    if bad.any():
        i = np.unravel_index(int(np.argmax(err - lim)), err.shape)
        raise AssertionError(f"{what}: max-abs {mx:.3e} over the bound at {i}: got {got[i]!r} "
                             f"ref {ref[i]!r} bound {np.broadcast_to(lim, err.shape)[i]:.3e}")
    assert mn <= mean_abs, f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}"
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


def with_wabs(fn, V, *args, v_index: int):
    """Run a row-wise oracle function whose values argument (position
    ``v_index`` in ``args``) is ``V`` on [V | |V|] (the value width follows
    V's), returning ``(o, lse, wabs)``: the output for V and, from the same
    softmax weights, their average of |V| (the compute term of a bf16
    output's bound)."""
    D = V.shape[-1]
    a = list(args)
    a.insert(v_index, np.concatenate([V, np.abs(V)], axis=-1))
    o, l = fn(*a)
    return o[..., :D], l, o[..., D:]
