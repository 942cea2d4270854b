"""GPU parity of the block-sparse forward (sa_attn_fwd_block_sparse) against the oracle.

The oracle is ``oracle.block_sparse_attention``: the page's pseudo-sparse run
(the block selection expanded into an element mask, then dense attention).
Tolerance as for the dense forward (tests/parity.py): ``5e-3 +
ulp_dtype(ref) / 2 + u * sum_j w_j |v_j|`` on out, 1e-3 on lse, -inf
matching -inf.  Block selections come from
``workloads.make_block_mask`` (sink and window blocks always, the rest at
random) or are built here for the edge cases.
"""
import numpy as np
import pytest
import torch

import online_softmax_amd as sa
import oracle
from parity import assert_lse_close, assert_out_close, out_bound, p_rounding, to_dev
from workloads import WORKLOADS, Workload, make_block_mask, make_inputs, to_f64

pytestmark = pytest.mark.gpu


def run_sparse(inp, bm):
    w = inp.w
    q, k, v, m, s = to_dev(inp)
    out, lse = sa.attn_fwd_block_sparse(q, k, v, bm.cuda(), causal=w.causal, scale=w.scale,
                                        key_padding_mask=m, alibi_slopes=s)
    torch.cuda.synchronize()
    return to_f64(out.cpu()), lse.cpu().double().numpy()


def ref_sparse(inp, bm, rows=None, abs_v=False):
    w = inp.w
    v = to_f64(inp.v)
    return oracle.block_sparse_attention(
        to_f64(inp.q), to_f64(inp.k), np.abs(v) if abs_v else v, w.scale, bm.numpy(), causal=w.causal,
        key_padding_mask=None if inp.mask is None else inp.mask.numpy(),
        alibi_slopes=None if inp.slopes is None else inp.slopes.numpy().astype(np.float64), rows=rows)


def check(inp, bm, rows=None, what=""):
    w = inp.w
    print(f"[sparse] {what or w.name} B={w.B} S_q={w.S_q} S_k={w.S_k} H={w.H_q}/{w.H_kv} D={w.D} "
          f"{w.dtype} causal={w.causal} mask={inp.mask is not None} alibi={inp.slopes is not None} "
          f"selected={bm.float().mean().item():.2f}", flush=True)
    out, lse = run_sparse(inp, bm)
    ref_o, ref_l = ref_sparse(inp, bm, rows)
    if rows is not None:
        out, lse = out[:, rows], lse[:, :, rows]
    dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    assert_out_close(out, ref_o, dt, what or w.name, p_rounding(ref_sparse(inp, bm, rows, abs_v=True)[0], dt))
    assert_lse_close(lse, ref_l, what or w.name)
    return out, lse


CASES = [
    Workload("sp_causal_d64", 2, 700, 700, 4, 2, 64, "fp16", causal=True, seed=80),
    Workload("sp_noncausal_d128", 1, 520, 390, 4, 4, 128, "bf16", seed=81),
    Workload("sp_all_features", 2, 600, 600, 8, 2, 128, "bf16", causal=True, alibi=True,
             random_tail=200, seed=82),
    Workload("sp_sq_lt_sk_causal", 1, 200, 900, 4, 1, 64, "fp16", causal=True, alibi=True, seed=83),
    Workload("sp_sq_gt_sk_causal", 1, 900, 300, 2, 2, 128, "fp16", causal=True, seed=84),
    Workload("sp_mask_alibi", 2, 384, 1000, 6, 3, 64, "bf16", alibi=True, random_tail=500, seed=85),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_sparse_cases(w):
    inp = make_inputs(w)
    check(inp, make_block_mask(w, keep=0.3))


@pytest.mark.parametrize("w", CASES[:3], ids=lambda w: w.name)
def test_sparse_all_selected_is_dense(w):
    """Every block selected: the dense forward's result (both against the oracle)."""
    inp = make_inputs(w)
    nbq, nbk = -(-w.S_q // 128), -(-w.S_k // 128)
    out, lse = check(inp, torch.ones((w.B, w.H_q, nbq, nbk), dtype=torch.uint8), what=w.name + " all")
    q, k, v, m, s = to_dev(inp)
    do, dl = sa.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, key_padding_mask=m, alibi_slopes=s)
    torch.cuda.synchronize()
    # The two sweeps visit the tiles in different orders (the dense one takes
    # the diagonal band first under causal ALiBi), so they agree to the sum
    # of their two distances from the oracle.
    dense = to_f64(do.cpu())
    dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    bm_all = torch.ones((w.B, w.H_q, nbq, nbk), dtype=torch.uint8)
    extra = p_rounding(ref_sparse(inp, bm_all, abs_v=True)[0], dt)
    assert (np.abs(out - dense) <= 2 * out_bound(dense, dt, extra)).all()
    assert np.abs(lse - dl.cpu().double().numpy()).max() <= 1e-4


def test_sparse_empty_and_diagonal_only():
    """A query block with nothing selected gives out = 0, lse = -inf; the
    diagonal-only selection is attention within each block."""
    w = Workload("sp_edges", 2, 512, 512, 4, 4, 64, "fp16", causal=True, seed=86)
    inp = make_inputs(w)
    bm = torch.zeros((2, 4, 4, 4), dtype=torch.uint8)
    for x in range(4):
        bm[:, :, x, x] = 1
    bm[1, 2, 3, :] = 0       # nothing for this block
    bm[0, 1, 0, :] = 0
    out, lse = check(inp, bm, what="diagonal only + empty")
    assert (out[1, 384:, 2] == 0).all() and np.isneginf(lse[1, 2, 384:]).all()
    assert (out[0, :128, 1] == 0).all() and np.isneginf(lse[0, 1, :128]).all()


def test_sparse_unselected_keys_do_not_leak():
    """Changing K/V in key blocks a query block did not select leaves its rows bit-identical."""
    w = Workload("sp_leak", 1, 1280, 1280, 4, 2, 128, "bf16", causal=True, alibi=True, seed=87)
    inp = make_inputs(w)
    bm = make_block_mask(w, keep=0.3)
    x = 9  # the last query block: no head of it selects key blocks 4 and 5
    bm[:, :, x, 4:6] = 0
    out1, lse1 = run_sparse(inp, bm)
    unused = [y for y in range(10) if not bm[0, :, x, y].any()]
    assert 4 in unused and 5 in unused
    k2, v2 = inp.k.clone(), inp.v.clone()
    for y in unused:
        k2[:, 128 * y:128 * (y + 1)] = torch.randn_like(k2[:, 128 * y:128 * (y + 1)].float()).to(k2.dtype)
        v2[:, 128 * y:128 * (y + 1)] = torch.randn_like(v2[:, 128 * y:128 * (y + 1)].float()).to(v2.dtype)
    inp.k, inp.v = k2, v2
    out2, lse2 = run_sparse(inp, bm)
    rows = slice(128 * x, 128 * (x + 1))
    assert np.array_equal(out1[:, rows], out2[:, rows]) and np.array_equal(lse1[:, :, rows], lse2[:, :, rows])
    # ... while rows of blocks that did select them change.
    assert not np.array_equal(out1[:, 640:768], out2[:, 640:768])


def _sample_rows(S, n, seed):
    base = {0, 1, 127, 128, 255, S // 2, S - 129, S - 128, S - 2, S - 1}
    rng = np.random.default_rng(seed)
    base |= set(rng.integers(0, S, n).tolist())
    return np.array(sorted(r for r in base if 0 <= r < S))


def test_config5_shape_sampled():
    """The 2 x 8192 x 32 x 128 bf16 causal ALiBi workload with its padding
    tails and a Stem-shaped selection, on sampled rows."""
    w = WORKLOADS["c5_alibi_8192"]
    inp = make_inputs(w)
    check(inp, make_block_mask(w), rows=_sample_rows(w.S_q, 12, 9), what="c5 block-sparse")


def test_sparse_deterministic():
    w = CASES[2]
    inp = make_inputs(w)
    bm = make_block_mask(w, keep=0.5)
    a, b = run_sparse(inp, bm), run_sparse(inp, bm)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_sparse_rejects_bad_mask():
    w = CASES[0]
    q, k, v, _, _ = to_dev(make_inputs(w))
    with pytest.raises(ValueError):
        sa.attn_fwd_block_sparse(q, k, v, torch.ones((2, 4, 5, 5), dtype=torch.uint8, device="cuda"))
