"""Helpers shared by the parity tests: tolerances and oracle calls on seeded inputs.

Tolerance (stated where it is used): an lse element passes when
``|gpu - oracle| <= 1e-3`` (with -inf matching -inf exactly) and an output
element when

    |gpu - oracle| <= 5e-3 + ulp_dtype(oracle) / 2 + u * sum_j w_j |v_j|

The 5e-3 / 1e-3 budget is the stated accuracy target for fp16/bf16 inputs.
The half-ulp term is the rounding of the exact result to the output dtype,
which alone exceeds 5e-3 for bf16 values of magnitude 2 or more and takes
most of it in [1, 2).  The last term is the rounding of each probability to
the input type before the P.V product (as the pages' kernels do, and as the
matrix cores require): it moves an output by at most u * sum_j w_j |v_j| (w
the row's softmax weights, u = 2^-8 for bfloat16, 2^-11 for float16).  Over
many keys these errors average out; over the few keys that carry a row's
weight under a steep ALiBi slope or a sparse mask they do not.  Every check
prints its maximum error, the count of elements above the literal 5e-3 and
its worst error / bound with and without the last term.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle.attention import _scores, _softmax_rows
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


def out_bound(ref, dtype, extra=None):
    """Per-element output bound: 5e-3 plus half an ulp of the output dtype at
    |ref|, plus ``extra`` (a further per-element term, see p_rounding)."""
    b = OUT_ATOL + half_ulp(ref, dtype)
    return b if extra is None else b + extra


def out_errors(gpu: np.ndarray, ref: np.ndarray, dtype: torch.dtype, extra=None):
    """(max abs error, count above the bound, count above 5e-3 literally,
    worst error / bound)."""
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    bound = out_bound(ref, dtype, extra)
    ratio = float((err / bound).max(initial=0.0))
    return float(err.max(initial=0.0)), int((err > bound).sum()), int((err > OUT_ATOL).sum()), ratio


def assert_out_close(gpu, ref, dtype, what="", extra=None):
    """``extra``: a further per-element term of the bound (see p_rounding)."""
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    mx, nbad, nlit, ratio = out_errors(gpu, ref, dtype, extra)
    plain = "" if extra is None else f" ({out_errors(gpu, ref, dtype)[3]:.3f} without the extra term)"
    print(f"    {what}: max|out err| {mx:.3e}, {nlit} of {gpu.size} above 5e-3, "
          f"worst err/bound {ratio:.3f}{plain}", flush=True)
    assert nbad == 0, f"{what}: {nbad} output elements beyond the bound (max abs err {mx:.3e})"


def p_rounding(abs_v_out, dtype):
    """u * sum_j w_j |v_j|: the bound on what rounding the probabilities to
    the input type before P.V moves an output (u = 2^-8 for bfloat16, 2^-11
    for float16).  ``abs_v_out`` is the oracle's output with |v| in place of
    v, i.e. sum_j w_j |v_j| per element."""
    u = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    return u * np.asarray(abs_v_out, np.float64)


def grad_rounding(inp, dout, dtype):
    """Per-element bound on what rounding the second products' operands to
    the input type moves the gradients: ``(u * scale * |dS| |k|,
    u * scale * |dS|^T |q|, u * P^T |dout|)`` for ``(dq, dk, dv)``, summed over
    the query heads of a key/value head like the gradients themselves.

    dS and P are the exact float64 ones of the backward's definition (the
    oracle's visibility, bias, score and softmax steps); rounding each dS or
    P element by at most u relative moves a product by at most u times the
    sum of the absolute terms.  u = 2^-8 for bfloat16, 2^-11 for float16."""
    w = inp.w
    q, k, v, do = to_f64(inp.q), to_f64(inp.k), to_f64(inp.v), np.asarray(dout, np.float64)
    G = w.H_q // w.H_kv
    u = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    eq, ek, ev = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(w.B):
        keep = oracle.visible(w.S_q, w.S_k, w.causal, None if inp.mask is None else inp.mask.numpy()[b])
        for h in range(w.H_q):
            hk = h // G
            bias = None if inp.slopes is None else oracle.alibi_bias(float(inp.slopes[h]), w.S_q, w.S_k)
            P, _ = _softmax_rows(_scores(q[b, :, h], k[b, :, hk], w.scale, keep, bias))
            dP = do[b, :, h] @ v[b, :, hk].T
            adS = np.abs(P * (dP - (P * dP).sum(axis=1, keepdims=True)))
            eq[b, :, h] = w.scale * (adS @ np.abs(k[b, :, hk]))
            ek[b, :, hk] += w.scale * (adS.T @ np.abs(q[b, :, h]))
            ev[b, :, hk] += P.T @ np.abs(do[b, :, h])
    return u * eq, u * ek, u * ev


def assert_lse_close(gpu, ref, what=""):
    gpu = np.asarray(gpu, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    ninf_r = np.isneginf(ref)
    assert (np.isneginf(gpu) == ninf_r).all(), f"{what}: -inf pattern of lse differs"
    assert not np.isnan(gpu).any(), f"{what}: NaN in lse"
    if (~ninf_r).any():
        err = np.abs(gpu[~ninf_r] - ref[~ninf_r]).max()
        assert err <= LSE_ATOL, f"{what}: lse max abs err {err:.3e} > {LSE_ATOL}"


def oracle_for(inp, rows=None, causal=None, abs_v=False):
    """Oracle (out, lse) for a workloads.Inputs bundle (optionally a row
    subset).  ``abs_v``: with |v| in place of v, so that out is
    sum_j w_j |v_j| per element (the scale of p_rounding)."""
    w = inp.w
    v = to_f64(inp.v)
    return oracle.attention(
        to_f64(inp.q), to_f64(inp.k), np.abs(v) if abs_v else v, w.scale,
        causal=w.causal if causal is None else causal,
        key_padding_mask=None if inp.mask is None else inp.mask.numpy(),
        alibi_slopes=None if inp.slopes is None else inp.slopes.numpy().astype(np.float64),
        rows=rows)


def to_dev(inp, device="cuda"):
    """Device copies of an Inputs bundle's tensors."""
    d = lambda t: None if t is None else t.to(device).contiguous()
    return d(inp.q), d(inp.k), d(inp.v), d(inp.mask), d(inp.slopes)
