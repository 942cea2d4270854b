"""GPU parity of the backward (sa_attn_bwd) against the float64 oracle.

The forward runs on the GPU first (its out and lse are the backward's
inputs, as in training); the oracle computes the exact gradients from the
same q, k, v and dout.  Tolerance: the "flash-attn-volta" page reports
dQ/dK/dV within 3e-3 max-abs of a float64 reference ("Backward
correctness", measured in float16 on a GPU without bfloat16); as for the
forward output, the bound here is ``atol + ulp_dtype(ref) / 2`` per element,
the half-ulp being the rounding of the exact gradient to the output dtype.

``atol`` is that 3e-3 for float16.  The error it bounds comes from rounding
the operands of the second products (dS and P) and the forward's output to
the input format, so it scales with the format's unit roundoff: bfloat16
keeps 8 significant bits against float16's 11, and its ``atol`` is
3e-3 * 2**3 = 2.4e-2.

The page's figure is a measured maximum at its shapes, not a bound that holds
at every size: a gradient of a key/value head sums the terms of all its query
heads and rows, and a dS or P term rounded to the input format moves it by up
to u times that term.  As for the forward output's probability term, the
bound adds ``u * sum |term|`` per element (``parity.grad_rounding``); the
forward output's own error, which enters through Di, stays within ``atol``.
At 8 query heads per key/value head (128 on 16) in bfloat16, the rounding
of dS, P and the output alone (emulated on the CPU in float64) takes dk and
dv past the plain ``atol + ulp/2`` by up to 1.5x.
"""
import dataclasses

import numpy as np
import pytest
import torch

import online_softmax_amd as sa
import oracle
from parity import grad_rounding, half_ulp, to_dev
from workloads import WORKLOADS, Inputs, Workload, make_dout, make_inputs, to_f64

pytestmark = pytest.mark.gpu
GRAD_ATOL = {"fp16": 3e-3, "bf16": 3e-3 * 2 ** 3}


def run_bwd(inp, dout_t):
    w = inp.w
    q, k, v, m, s = to_dev(inp)
    out, lse = sa.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, key_padding_mask=m, alibi_slopes=s)
    dq, dk, dv = sa.attn_bwd(q, k, v, out, dout_t.cuda(), lse, causal=w.causal, scale=w.scale,
                             key_padding_mask=m, alibi_slopes=s)
    torch.cuda.synchronize()
    return dq, dk, dv


def check(inp, what=""):
    w = inp.w
    print(f"[bwd] {what or w.name} B={w.B} S_q={w.S_q} S_k={w.S_k} H={w.H_q}/{w.H_kv} D={w.D} "
          f"{w.dtype} causal={w.causal} mask={inp.mask is not None} alibi={inp.slopes is not None}",
          flush=True)
    dout = make_dout(w)
    got = run_bwd(inp, dout)
    compare(inp, dout, got, what)
    return got


def compare(inp, dout, got, what=""):
    """dq, dk, dv of the GPU (``got``) against the oracle's, element by element."""
    w = inp.w
    ref = oracle.attention_bwd(to_f64(inp.q), to_f64(inp.k), to_f64(inp.v), to_f64(dout), w.scale,
                               causal=w.causal,
                               key_padding_mask=None if inp.mask is None else inp.mask.numpy(),
                               alibi_slopes=None if inp.slopes is None else inp.slopes.numpy())
    dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    extra = grad_rounding(inp, to_f64(dout), dt)
    for name, g, r, x in zip(("dq", "dk", "dv"), got, ref, extra):
        g = to_f64(g.cpu())
        assert np.isfinite(g).all(), f"{what or w.name}: non-finite {name}"
        err = np.abs(g - r)
        plain = GRAD_ATOL[w.dtype] + half_ulp(r, dt)
        bound = plain + x
        print(f"    {name}: max abs err {err.max(initial=0):.3e}  max |ref| {np.abs(r).max(initial=0):.3e}  "
              f"worst err/bound {np.max(err / bound, initial=0):.3f} "
              f"({np.max(err / plain, initial=0):.3f} without the rounding term)", flush=True)
        assert (err <= bound).all(), f"{what or w.name}: {int((err > bound).sum())} {name} elements beyond bound"


CASES = [
    Workload("b_plain", 1, 128, 128, 2, 2, 64, "fp16", seed=60),
    Workload("b_causal_d128", 2, 200, 200, 4, 2, 128, "bf16", causal=True, seed=61),
    Workload("b_mask_sq_lt_sk", 1, 150, 333, 4, 4, 64, "fp16", random_tail=200, seed=62),
    Workload("b_alibi_causal", 1, 260, 260, 8, 8, 128, "bf16", causal=True, alibi=True, seed=63),
    Workload("b_all_features", 2, 300, 300, 8, 2, 128, "bf16", causal=True, alibi=True,
             random_tail=64, seed=64),
    Workload("b_sq_lt_sk_causal", 1, 77, 300, 4, 4, 64, "fp16", causal=True, seed=65),
    Workload("b_sq_gt_sk_causal", 1, 300, 77, 4, 4, 64, "fp16", causal=True, seed=66),
    Workload("b_gqa7_alibi", 2, 129, 129, 14, 2, 64, "fp16", alibi=True, seed=67),
    Workload("b_s1000_mask", 1, 1000, 1000, 2, 2, 64, "bf16", causal=True, random_tail=300, seed=68),
    Workload("b_alibi_noncausal", 1, 190, 190, 4, 4, 128, "fp16", alibi=True, seed=69),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_bwd_cases(w):
    check(make_inputs(w))


def test_bwd_config2_full():
    check(make_inputs(WORKLOADS["c2_causal_pad16"]))


@pytest.mark.parametrize("w", [
    # 8 query heads per key/value head: dk and dv sum 8 heads x 300 rows; ragged ends, padding, ALiBi
    Workload("b_gqa8_causal_all", 4, 300, 300, 128, 16, 64, "bf16", causal=True, alibi=True, random_tail=60,
             seed=75),
    # 8 query heads per key/value head, queries shorter than keys
    Workload("b_gqa8_plain", 2, 300, 340, 64, 8, 64, "fp16", seed=76),
], ids=lambda w: w.name)
def test_bwd_large_gqa(w):
    """Grids of many workgroups, with large query-head groups per key/value
    head; checked in full."""
    check(make_inputs(w))


@pytest.mark.parametrize("name,heads", [("c3_causal_4096", [(0, 0), (0, 11)]),
                                        ("c5_alibi_8192", [(0, 0), (1, 29)])])
def test_bwd_full_size_sampled_heads(name, heads):
    """The backward at the benchmark's full sizes, in the launch configuration
    it times: the gradients of a few (batch, head) slices checked in full
    against the oracle run on that slice alone.  These shapes have as many
    key/value heads as query heads, so a key/value head's dk and dv come from
    its one query head; the slice carries its batch row's padding and its
    head's ALiBi slope."""
    w = WORKLOADS[name]
    assert w.H_q == w.H_kv
    inp = make_inputs(w)
    dout = make_dout(w)
    print(f"[bwd] {name} full size B={w.B} S={w.S_q} H={w.H_q} D={w.D} {w.dtype}; heads {heads}", flush=True)
    got = [g.cpu() for g in run_bwd(inp, dout)]
    for b, h in heads:
        one = lambda t: t[b:b + 1, :, h:h + 1].contiguous()
        sub = Inputs(dataclasses.replace(w, B=1, H_q=1, H_kv=1), one(inp.q), one(inp.k), one(inp.v),
                     None if inp.mask is None else inp.mask[b:b + 1].contiguous(),
                     None if inp.slopes is None else inp.slopes[h:h + 1].contiguous())
        print(f"  slice b={b} h={h}", flush=True)
        compare(sub, one(dout), [one(g) for g in got], f"{name} b={b} h={h}")


def test_bwd_empty_rows_and_keys():
    w = Workload("b_empty", 1, 64, 64, 2, 2, 64, "fp16", seed=70)
    inp = make_inputs(w)
    q, k, v, _, _ = to_dev(inp)
    # No query rows: dk = dv = 0.
    q0 = q[:, :0].contiguous()
    dq, dk, dv = sa.attn_bwd(q0, k, v, q0.clone(), q0.clone(),
                             torch.empty((1, 2, 0), device="cuda"), dk=torch.full_like(k, 7), dv=torch.full_like(v, 7))
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()
    # No keys: dq = 0.
    k0, v0 = k[:, :0].contiguous(), v[:, :0].contiguous()
    out, lse = sa.attn_fwd(q, k0, v0)
    dq, dk, dv = sa.attn_bwd(q, k0, v0, out, torch.ones_like(q), lse, dq=torch.full_like(q, 7))
    torch.cuda.synchronize()
    assert (dq == 0).all()


def test_bwd_fully_masked_batch_row():
    w = Workload("b_masked_row", 2, 100, 100, 2, 2, 64, "fp16", seed=71)
    inp = make_inputs(w)
    inp.mask = torch.ones((2, 100), dtype=torch.uint8)
    inp.mask[1] = 0
    dq, dk, dv = check(inp, "fully masked batch row")
    assert (dq[1] == 0).all() and (dk[1] == 0).all() and (dv[1] == 0).all()


def test_bwd_deterministic():
    inp = make_inputs(Workload("b_det", 1, 300, 300, 4, 2, 128, "bf16", causal=True, alibi=True,
                               random_tail=50, seed=72))
    dout = make_dout(inp.w)
    a, b = run_bwd(inp, dout), run_bwd(inp, dout)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_bwd_causal_leak_bitwise():
    """dq of row i is bit-identical when keys and values after i change (the
    causal-leak check of the "flash-attn-volta" page)."""
    w = Workload("b_leak", 1, 256, 256, 4, 4, 64, "fp16", causal=True, seed=73)
    inp = make_inputs(w)
    dout = make_dout(w)
    dq1, _, _ = run_bwd(inp, dout)
    cut = 100
    inp.k[:, cut + 1:] = torch.randn_like(inp.k[:, cut + 1:].float()).to(inp.k.dtype)
    inp.v[:, cut + 1:] = torch.randn_like(inp.v[:, cut + 1:].float()).to(inp.v.dtype)
    dq2, _, _ = run_bwd(inp, dout)
    assert torch.equal(dq1[:, :cut + 1], dq2[:, :cut + 1])
    assert not torch.equal(dq1[:, cut + 1:], dq2[:, cut + 1:])


def test_bwd_paired_causal_grid():
    """A causal grid of exactly two workgroups per CU for both kernels
    (B * H * 4 blocks of 128 = 512 on a 256-CU device), where workgroups j
    and j + CUs take complementary blocks of one head; checked in full."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    w = Workload("b_pair_grid", 2, 512, 512, 64, 64, 128, "fp16", causal=True, seed=74)
    print(f"[bwd] {w.B * w.H_q * 4} query blocks and {w.B * w.H_kv * 4} key blocks on {ncu} CUs", flush=True)
    check(make_inputs(w))
