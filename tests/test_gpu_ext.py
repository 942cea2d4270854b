"""GPU parity of the extended forward (sa_attn_fwd_ext: additive float mask
and Philox dropout) against the oracle ``oracle.attention_ext``.

Tolerance as for the plain forward (tests/parity.py): ``5e-3 +
ulp_dtype(ref) / 2 + u * sum_j w_j |v_j|`` on out, 1e-3 on lse, -inf matching
-inf.  The dropout decisions are integer
comparisons of Philox words on both sides, so the dropped outputs are
compared element by element like any other.  With dropout the product P V
sums each kept probability, rounded to the input type (relative error at
most u = 2^-8 for bfloat16, 2^-11 for float16), times 1 / (1 - p): the
rounding error of an output is then at most u max|v| / (1 - p), and the
absolute part of the bound becomes ``max(5e-3, u max|v|) / (1 - p)``.
"""
import dataclasses

import numpy as np
import pytest
import torch

import online_softmax_amd as sa
import oracle
from parity import OUT_ATOL, assert_lse_close, assert_out_close, out_bound, p_rounding, to_dev
from workloads import WORKLOADS, Workload, make_bias, make_inputs, to_f64

pytestmark = pytest.mark.gpu


def run_ext(inp, bias=None, p=0.0, seed=0, offset=0):
    w = inp.w
    q, k, v, m, s = to_dev(inp)
    out, lse = sa.attn_fwd_ext(q, k, v, causal=w.causal, scale=w.scale, key_padding_mask=m,
                               alibi_slopes=s, attn_bias=None if bias is None else bias.cuda(),
                               dropout_p=p, seed=seed, offset=offset)
    torch.cuda.synchronize()
    return to_f64(out.cpu()), lse.cpu().double().numpy()


def ref_ext(inp, bias=None, p=0.0, seed=0, offset=0, rows=None):
    w = inp.w
    return oracle.attention_ext(
        to_f64(inp.q), to_f64(inp.k), to_f64(inp.v), w.scale, causal=w.causal,
        key_padding_mask=None if inp.mask is None else inp.mask.numpy(),
        alibi_slopes=None if inp.slopes is None else inp.slopes.numpy().astype(np.float64),
        attn_bias=None if bias is None else bias.double().numpy(), dropout_p=p, seed=seed,
        offset=offset, rows=rows)


def check(inp, bias=None, p=0.0, seed=0, offset=0, rows=None, what=""):
    w = inp.w
    print(f"[ext] {what or w.name} B={w.B} S_q={w.S_q} S_k={w.S_k} H={w.H_q}/{w.H_kv} D={w.D} "
          f"{w.dtype} causal={w.causal} mask={inp.mask is not None} alibi={inp.slopes is not None} "
          f"bias={None if bias is None else tuple(bias.shape)} p={p} seed={seed} offset={offset}", flush=True)
    out, lse = run_ext(inp, bias, p, seed, offset)
    ref_o, ref_l = ref_ext(inp, bias, p, seed, offset, rows)
    if rows is not None:
        out, lse = out[:, rows], lse[:, :, rows]
    dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    if p > 0.0:
        u = 2.0 ** -8 if w.dtype == "bf16" else 2.0 ** -11
        atol = max(OUT_ATOL, u * float(inp.v.float().abs().max())) / (1.0 - p)
        err = np.abs(out - ref_o)
        bound = out_bound(ref_o, dt) - OUT_ATOL + atol
        print(f"    dropout bound {atol:.3e} + half-ulp; max err {err.max():.3e}; "
              f"worst err/bound {(err / bound).max():.3f}", flush=True)
        assert np.isfinite(out).all() and (err <= bound).all(), f"{what or w.name}: {(err > bound).sum()} beyond"
    else:
        extra = p_rounding(ref_ext(dataclasses.replace(inp, v=inp.v.abs()), bias, p, seed, offset, rows)[0], dt)
        assert_out_close(out, ref_o, dt, what or w.name, extra)
    assert_lse_close(lse, ref_l, what or w.name)
    return out, lse


CASES = [
    # workload, bias kind (None = no bias), dropout p
    (Workload("ex_bias_bhqk", 2, 300, 300, 4, 2, 64, "fp16", causal=True, seed=90), "bhqk", 0.0),
    (Workload("ex_bias_b1qk_alibi", 1, 260, 390, 8, 8, 128, "bf16", alibi=True, seed=91), "b1qk", 0.0),
    (Workload("ex_bias_qk_ragged", 2, 129, 201, 4, 4, 64, "bf16", causal=True, random_tail=50, seed=92), "qk", 0.0),
    (Workload("ex_bias_b11k", 2, 200, 333, 6, 3, 128, "fp16", seed=93), "b11k", 0.0),
    (Workload("ex_drop", 2, 256, 256, 4, 2, 64, "fp16", causal=True, seed=94), None, 0.1),
    (Workload("ex_drop_half_all", 2, 300, 300, 8, 2, 128, "bf16", causal=True, alibi=True,
              random_tail=100, seed=95), None, 0.5),
    (Workload("ex_bias_drop", 1, 400, 400, 4, 4, 128, "fp16", causal=True, alibi=True, seed=96), "b1qk", 0.2),
    (Workload("ex_bias_drop_sq_lt_sk", 1, 100, 500, 2, 1, 64, "bf16", causal=True, random_tail=40, seed=97),
     "bhqk", 0.3),
]


@pytest.mark.parametrize("w,kind,p", CASES, ids=lambda c: c.name if isinstance(c, Workload) else str(c))
def test_ext_cases(w, kind, p):
    inp = make_inputs(w)
    bias = None if kind is None else make_bias(w, kind)
    check(inp, bias, p, seed=0x123456789ABC + w.seed, offset=w.seed)


def test_ext_plain_matches_forward():
    """No bias, no dropout: the plain forward's result."""
    w = Workload("ex_plain", 2, 300, 300, 4, 2, 128, "bf16", causal=True, alibi=True, random_tail=60, seed=98)
    inp = make_inputs(w)
    out, lse = check(inp)
    q, k, v, m, s = to_dev(inp)
    o2, l2 = sa.attn_fwd(q, k, v, causal=True, scale=w.scale, key_padding_mask=m, alibi_slopes=s)
    torch.cuda.synchronize()
    assert np.abs(lse - l2.cpu().double().numpy()).max() <= 1e-4


def test_ext_dropout_determinism_and_lse():
    w = Workload("ex_det", 1, 256, 256, 4, 4, 64, "fp16", causal=True, seed=99)
    inp = make_inputs(w)
    a = run_ext(inp, None, 0.3, seed=7, offset=1)
    b = run_ext(inp, None, 0.3, seed=7, offset=1)
    c = run_ext(inp, None, 0.3, seed=7, offset=2)
    d = run_ext(inp, None, 0.6, seed=8)
    e = run_ext(inp, None, 0.0)   # the plain forward's kernel
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0])
    # lse is that of the softmax before dropout: the same bits for any p,
    # seed and offset, and the plain forward's up to rounding order.
    assert np.array_equal(a[1], c[1]) and np.array_equal(a[1], d[1])
    assert np.abs(a[1] - e[1]).max() <= 1e-5


def test_ext_neg_inf_bias_row():
    """A row whose bias hides every key gives out = 0 and lse = -inf."""
    w = Workload("ex_ninf", 1, 130, 140, 2, 2, 64, "fp16", seed=100)
    inp = make_inputs(w)
    bias = make_bias(w, "bhqk", ninf=0.0)
    bias[0, 1, 5, :] = float("-inf")
    bias[0, 0, 129, :] = float("-inf")
    out, lse = check(inp, bias, what="rows hidden by the bias")
    assert (out[0, 5, 1] == 0).all() and np.isneginf(lse[0, 1, 5])
    assert (out[0, 129, 0] == 0).all() and np.isneginf(lse[0, 0, 129])


def _sample_rows(S, n, seed):
    base = {0, 1, 63, 64, 127, 128, S // 2, S - 65, S - 2, S - 1}
    rng = np.random.default_rng(seed)
    base |= set(rng.integers(0, S, n).tolist())
    return np.array(sorted(r for r in base if 0 <= r < S))


def test_config3_shape_bias_dropout_sampled():
    """The 1 x 4096 x 16 x 128 causal workload with a [1, 1, 4096, 4096] bias
    and dropout 0.1, on sampled rows."""
    w = WORKLOADS["c3_causal_4096"]
    inp = make_inputs(w)
    check(inp, make_bias(w, "b1qk"), 0.1, seed=2024, offset=3, rows=_sample_rows(w.S_q, 12, 4),
          what="c3 causal + bias + dropout")


def test_ext_rejects():
    w = CASES[0][0]
    q, k, v, _, _ = to_dev(make_inputs(w))
    for p in (-0.1, 1.0):
        with pytest.raises(sa.SaAttnError):
            sa.attn_fwd_ext(q, k, v, dropout_p=p)
    with pytest.raises(ValueError):
        sa.attn_fwd_ext(q, k, v, attn_bias=torch.zeros(3, 3, device="cuda"))


@pytest.mark.parametrize("w,p", [
    (Workload("keep_f16_d128", 2, 300, 128, 4, 2, 128, "fp16", seed=170), 0.3),
    (Workload("keep_bf16_d64_causal", 2, 200, 64, 6, 3, 64, "bf16", causal=True, seed=171), 0.5),
    (Workload("keep_bf16_d128_mask_alibi", 1, 260, 120, 4, 4, 128, "bf16", causal=True, alibi=True,
              random_tail=20, seed=172), 0.1),
], ids=lambda c: c.name if isinstance(c, Workload) else str(c))
def test_dropout_keep_pattern_exact(w, p):
    """The dropout decisions, bit for bit.  With one-hot values (v_j = e_j,
    S_k <= D) output column j of row i is P[i, j] * keep[i, j] / (1 - p): it
    is zero exactly where the kernel dropped the probability (or the key is
    hidden), so the zero pattern of out[..., :S_k] is compared element by
    element with the oracle's Philox rule (oracle.philox.keep_mask)."""
    inp = make_inputs(w)
    v = torch.zeros_like(inp.v)
    for j in range(w.S_k):
        v[:, j, :, j] = 1.0
    inp.v = v
    seed, offset = 0x0123456789ABCDEF + w.seed, 7 * w.seed
    out, lse = run_ext(inp, None, p, seed=seed, offset=offset)
    ref_o, ref_l = ref_ext(inp, None, p, seed=seed, offset=offset)
    nz = out[..., :w.S_k] != 0                                 # [B, S_q, H_q, S_k]
    assert (out[..., w.S_k:] == 0).all()
    mism = 0
    for b in range(w.B):
        vis = oracle.visible(w.S_q, w.S_k, w.causal, None if inp.mask is None else inp.mask[b].numpy())
        for h in range(w.H_q):
            keep = oracle.philox.keep_mask(b, h, w.H_q, np.arange(w.S_q), w.S_k, p, seed, offset)
            mism += int((nz[b, :, h, :] != (keep & vis)).sum())
    frac = float(nz.mean())
    print(f"[ext] {w.name}: p={p}, {mism} keep decisions differ, nonzero fraction {frac:.3f}", flush=True)
    assert mism == 0
    # And the values themselves, to the dropout bound.
    check(inp, None, p, seed=seed, offset=offset, what=w.name + " values")
