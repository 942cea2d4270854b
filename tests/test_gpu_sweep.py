"""Seeded sweep of every compiled instance against the oracle.

Each entry point (forward, backward, block-sparse, extended, decode) is
built for {float16, bfloat16} x D {64, 128} x {causal} x {key-padding mask}
x {ALiBi} (decode: no causal rule).  For every combination one shape is drawn
from a seeded generator (batch, query heads per key/value head, ragged
query and key lengths, masked tail lengths up to all the keys) and the
whole output is compared with the oracle, to the same bounds as the other
parity tests.  The shapes are small, so the forwards take the four-wave and
two-group kernels; the eight-wave and persistent ones have their own tests.
"""
import itertools

import numpy as np
import pytest
import torch

import online_softmax_amd as sa
import test_gpu_bwd as bwd
import test_gpu_decode as dec
import test_gpu_ext as ext
import test_gpu_fwd as fwd
import test_gpu_sparse as sparse
from parity import assert_lse_close, assert_out_close, oracle_for, p_rounding
from workloads import Workload, make_bias, make_block_mask, make_inputs

pytestmark = pytest.mark.gpu

COMBOS = list(itertools.product(("fp16", "bf16"), (64, 128), (False, True), (False, True), (False, True)))


def _cid(c):
    dt, D, causal, mask, alibi = c
    return f"{dt}_d{D}" + "_causal" * causal + "_mask" * mask + "_alibi" * alibi


KIND = {"fwd": 1, "bwd": 2, "sparse": 3, "ext": 4}


def _shape(kind, i, c, max_s, groups, max_b=3, max_hkv=3):
    dt, D, causal, mask, alibi = c
    r = np.random.default_rng([KIND[kind], i])
    B = int(r.integers(1, max_b + 1))
    H_kv = int(r.integers(1, max_hkv + 1))
    G = int(r.choice(groups))
    S_q = int(r.integers(1, max_s + 1))
    S_k = int(r.integers(1, max_s + 1))
    tail = int(r.integers(1, S_k + 1)) if mask else 0
    return Workload(f"{kind}_{i}_{_cid(c)}", B, S_q, S_k, H_kv * G, H_kv, D, dt, causal=causal, alibi=alibi,
                    random_tail=tail, seed=3000 + 100 * KIND[kind] + i)


@pytest.mark.parametrize("i,c", list(enumerate(COMBOS)), ids=[_cid(c) for c in COMBOS])
def test_sweep_forward(i, c):
    fwd.check(make_inputs(_shape("fwd", i, c, 350, (1, 2, 3, 5, 7))))


@pytest.mark.parametrize("i,c", list(enumerate(COMBOS)), ids=[_cid(c) for c in COMBOS])
def test_sweep_backward(i, c):
    bwd.check(make_inputs(_shape("bwd", i, c, 200, (1, 2, 3), max_b=2, max_hkv=2)))


@pytest.mark.parametrize("i,c", list(enumerate(COMBOS)), ids=[_cid(c) for c in COMBOS])
def test_sweep_block_sparse(i, c):
    w = _shape("sparse", i, c, 400, (1, 2, 4))
    sparse.check(make_inputs(w), make_block_mask(w, keep=0.3))


@pytest.mark.parametrize("i,c", list(enumerate(COMBOS)), ids=[_cid(c) for c in COMBOS])
def test_sweep_extended(i, c):
    """The extended forward with a seeded additive mask at one of its four
    broadcast shapes and/or dropout (at least one of them, else the call is
    the plain forward's)."""
    w = _shape("ext", i, c, 300, (1, 2, 3))
    r = np.random.default_rng([KIND["ext"], 100 + i])
    kind = [None, "bhqk", "b1qk", "qk", "b11k"][int(r.integers(0, 5))]
    p = [0.0, 0.15, 0.4][int(r.integers(0, 3))]
    if kind is None and p == 0.0:
        p = 0.15
    ext.check(make_inputs(w), None if kind is None else make_bias(w, kind), p, seed=0x5EED0000 + i, offset=i)


DEC_COMBOS = [c for c in COMBOS if not c[2]]  # one query row: the causal rule hides nothing


@pytest.mark.parametrize("i,c", list(enumerate(DEC_COMBOS)), ids=[_cid(c) for c in DEC_COMBOS])
def test_sweep_decode(i, c):
    """Both decode entry points: the split and merge launches and the single
    kernel (up to 20 query heads per key/value head, so two head groups)."""
    dt, D, _, mask, alibi = c
    r = np.random.default_rng([7, i])
    B = int(r.integers(1, 5))
    H_kv = int(r.integers(1, 4))
    G = int(r.choice((1, 2, 7, 8, 16, 20)))
    S_k = int(r.integers(1, 5001))
    tail = int(r.integers(1, S_k + 1)) if mask else 0
    w = Workload(f"dec_{i}_{_cid(c)}", B, 1, S_k, H_kv * G, H_kv, D, dt, alibi=alibi, random_tail=tail,
                 seed=3500 + i)
    inp = make_inputs(w)
    dec.check(inp)
    out, lse = dec.run_fused(inp, sa.decode_fused_workspace(w.B, w.H_q, w.S_k, w.D, "cuda"))
    dtt = torch.float16 if dt == "fp16" else torch.bfloat16
    assert_out_close(out, oracle_for(inp, causal=False)[0], dtt, w.name + " (single kernel)",
                     p_rounding(oracle_for(inp, causal=False, abs_v=True)[0], dtt))
    assert_lse_close(lse, oracle_for(inp, causal=False)[1], w.name + " (single kernel)")
