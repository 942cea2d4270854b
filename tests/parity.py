"""Helpers shared by the parity tests: tolerances and oracle calls on seeded inputs.

Tolerance (stated where it is used): an output element passes when
``|gpu - oracle| <= 5e-3 + ulp_dtype(oracle) / 2`` and an lse element when
``|gpu - oracle| <= 1e-3`` (with -inf matching -inf exactly).  The 5e-3 / 1e-3
budget is the stated accuracy target for fp16/bf16 inputs; the half-ulp term
is the rounding of the exact result to the output dtype, which alone exceeds
5e-3 for bf16 values of magnitude 2 or more.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import to_f64

OUT_ATOL = 5e-3
LSE_ATOL = 1e-3


def half_ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Half a unit in the last place of fp16/bf16 at the magnitude of x."""
    mant, min_exp = (10, -14) if dtype == torch.float16 else (7, -126)
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, min_exp)
    return 0.5 * np.exp2(e - mant)


def out_errors(gpu: np.ndarray, ref: np.ndarray, dtype: torch.dtype, extra=None):
    """(max abs error, count above the bound, count above 5e-3 literally)."""
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    bound = OUT_ATOL + half_ulp(ref, dtype) + (0.0 if extra is None else extra)
    return float(err.max(initial=0.0)), int((err > bound).sum()), int((err > OUT_ATOL).sum())


def assert_out_close(gpu, ref, dtype, what="", extra=None):
    """``extra``: a further per-element term of the bound (see p_rounding)."""
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    mx, nbad, _ = out_errors(gpu, ref, dtype, extra)
    assert nbad == 0, f"{what}: {nbad} output elements beyond the bound (max abs err {mx:.3e})"


def p_rounding(abs_v_out, dtype):
    """The rounding of each probability to the input type before P.V moves an
    output by at most u * sum_j w_j |v_j| (w the row's softmax weights; u =
    2^-9 for bfloat16, 2^-12 for float16).  Over many keys these errors
    average out and the plain bound holds; where a row's weight sits on a few
    keys (a steep ALiBi slope decays it by a constant factor per key, or few
    keys are visible) they do not.  ``abs_v_out`` is the oracle's output with
    |v| in place of v, i.e. sum_j w_j |v_j| per element."""
    u = 2.0 ** -9 if dtype == torch.bfloat16 else 2.0 ** -12
    return u * np.asarray(abs_v_out, np.float64)


def assert_lse_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    ninf_r = np.isneginf(ref)
    assert (np.isneginf(gpu) == ninf_r).all(), f"{what}: -inf pattern of lse differs"
    assert not np.isnan(gpu).any(), f"{what}: NaN in lse"
    if (~ninf_r).any():
        err = np.abs(gpu[~ninf_r] - ref[~ninf_r]).max()
        assert err <= LSE_ATOL, f"{what}: lse max abs err {err:.3e} > {LSE_ATOL}"


def oracle_for(inp, rows=None, causal=None):
    """Oracle (out, lse) for a workloads.Inputs bundle (optionally a row subset)."""
    w = inp.w
    return oracle.attention(
        to_f64(inp.q), to_f64(inp.k), to_f64(inp.v), w.scale,
        causal=w.causal if causal is None else causal,
        key_padding_mask=None if inp.mask is None else inp.mask.numpy(),
        alibi_slopes=None if inp.slopes is None else inp.slopes.numpy().astype(np.float64),
        rows=rows)


def to_dev(inp, device="cuda"):
    """Device copies of an Inputs bundle's tensors."""
    d = lambda t: None if t is None else t.to(device).contiguous()
    return d(inp.q), d(inp.k), d(inp.v), d(inp.mask), d(inp.slopes)
