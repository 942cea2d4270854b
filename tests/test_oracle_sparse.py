"""Pins of the block-sparse oracle (``oracle.block_sparse_attention``).

The oracle restricts each block of query rows to its selected key blocks
(the "Stem" page, section 2.3, "Block-Sparse Attention"; block size 128 from
its section 6).  It is checked against facts that do not go through its own
code path:

* torch's scaled_dot_product_attention in float64 with an element mask built
  here by explicit loops over (row, key);
* the scalar brute force of ``oracle.brute`` with the same block rule;
* a block-diagonal selection, which is independent dense attention on each
  block (torch, one block at a time);
* keys in blocks that a query block did not select have no influence on its
  rows (their outputs and lse stay bit-identical when those keys change);
* an all-selected mask is the dense definition; a query block that selects
  nothing gets out = 0 and lse = -inf.

A mutation test plants plausible mistakes in the oracle (on the CPU) and
checks that the pins reject each.
"""
import importlib

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

oatt = importlib.import_module("oracle.attention")


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def random_blocks(rng, B, H, nbq, nbk, p=0.5):
    return (rng.random((B, H, nbq, nbk)) < p).astype(np.uint8)


def element_mask(bm_bh, S_q, S_k, block, causal, pad_row):
    """keep[i, j] by explicit loops."""
    keep = np.zeros((S_q, S_k), dtype=bool)
    for i in range(S_q):
        for j in range(S_k):
            ok = bool(bm_bh[i // block][j // block])
            if causal and j > i + S_k - S_q:
                ok = False
            if pad_row is not None and not pad_row[j]:
                ok = False
            keep[i, j] = ok
    return keep


def sdpa_ref(q, k, v, scale, bm, block, causal, mask, slopes):
    """torch float64 reference: bias + explicit element mask; rows with no key -> 0, -inf."""
    B, S_q, H_q, D = q.shape
    S_k, H_kv = k.shape[1], k.shape[2]
    G = H_q // H_kv
    out = np.zeros((B, S_q, H_q, D))
    lse = np.full((B, H_q, S_q), -np.inf)
    for b in range(B):
        for h in range(H_q):
            keep = element_mask(bm[b, h], S_q, S_k, block, causal, None if mask is None else mask[b])
            qt = torch.from_numpy(q[b, :, h, :])
            kt = torch.from_numpy(k[b, :, h // G, :])
            vt = torch.from_numpy(v[b, :, h // G, :])
            bias = torch.zeros(S_q, S_k, dtype=torch.float64)
            if slopes is not None:
                i = torch.arange(S_q, dtype=torch.float64)[:, None] + (S_k - S_q)
                j = torch.arange(S_k, dtype=torch.float64)[None, :]
                bias = -float(slopes[h]) * (i - j).abs()
            km = torch.from_numpy(keep)
            attn = torch.where(km, bias, torch.tensor(float("-inf"), dtype=torch.float64))
            rows = km.any(dim=1)
            if rows.any():
                o = torch.nn.functional.scaled_dot_product_attention(
                    qt[rows][None], kt[None], vt[None], attn_mask=attn[rows][None], scale=float(scale))[0]
                out[b, rows.numpy(), h, :] = o.numpy()
                s = float(scale) * (qt @ kt.T) + attn
                lse[b, h, rows.numpy()] = torch.logsumexp(s[rows], dim=1).numpy()
    return out, lse


def close(a, b, tol=1e-10):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape:
        return False
    fin = np.isfinite(b)
    return bool(np.array_equal(np.isfinite(a), fin) and np.all(a[~fin] == b[~fin])
                and np.all(np.abs(a[fin] - b[fin]) <= tol * (1 + np.abs(b[fin]))))


CASES = [
    # B, S_q, S_k, H_q, H_kv, D, block, causal, mask, alibi, seed
    (2, 9, 9, 4, 2, 4, 2, True, False, False, 1),
    (1, 7, 11, 2, 1, 3, 2, True, True, True, 2),
    (2, 10, 6, 2, 2, 4, 3, False, True, False, 3),
    (1, 8, 8, 4, 4, 2, 4, False, False, True, 4),
    (1, 12, 12, 2, 1, 4, 3, True, False, True, 5),
]
# At the page's block size of 128: three query and three key blocks, ragged.
CASE_128 = (1, 300, 300, 2, 1, 8, 128, True, True, True, 6)


def make_case(c, p=0.5):
    B, S_q, S_k, H_q, H_kv, D, blk, causal, use_mask, use_alibi, seed = c
    rng = np.random.default_rng(seed)
    q, k, v = rnd(rng, B, S_q, H_q, D), rnd(rng, B, S_k, H_kv, D), rnd(rng, B, S_k, H_kv, D)
    nbq, nbk = -(-S_q // blk), -(-S_k // blk)
    bm = random_blocks(rng, B, H_q, nbq, nbk, p)
    mask = None
    if use_mask:
        mask = np.ones((B, S_k), np.uint8)
        mask[:, -2:] = 0
        mask[0, 1] = 0
    slopes = rng.uniform(0.1, 1.0, H_q) if use_alibi else None
    return q, k, v, 0.6, bm, blk, causal, mask, slopes


def call(fn, q, k, v, scale, bm, blk, causal, mask, slopes):
    return fn(q, k, v, scale, bm, causal=causal, key_padding_mask=mask, alibi_slopes=slopes, block=blk)


# ------------------------------------------------------------------ pins

def pin_sdpa(fn):
    for c in CASES + [CASE_128]:
        args = make_case(c)
        o, l = call(fn, *args)
        ro, rl = sdpa_ref(*args)
        assert close(o, ro) and close(l, rl), c


def pin_brute(fn):
    for c in CASES[:3]:
        q, k, v, sc, bm, blk, causal, mask, slopes = make_case(c)
        o, l = call(fn, q, k, v, sc, bm, blk, causal, mask, slopes)
        bo, bl = brute.attention(q.tolist(), k.tolist(), v.tolist(), sc, causal,
                                 None if mask is None else mask.tolist(),
                                 None if slopes is None else slopes.tolist(), bm.tolist(), blk)
        assert close(o, np.array(bo)) and close(l, np.array(bl)), c


def pin_block_diagonal(fn):
    rng = np.random.default_rng(11)
    B, S, H, D, blk = 1, 12, 2, 4, 4
    q, k, v = rnd(rng, B, S, H, D), rnd(rng, B, S, H, D), rnd(rng, B, S, H, D)
    bm = np.zeros((B, H, 3, 3), np.uint8)
    for x in range(3):
        bm[:, :, x, x] = 1
    o, l = fn(q, k, v, 0.5, bm, block=blk)
    for h in range(H):
        for x in range(3):
            sl = slice(blk * x, blk * (x + 1))
            qt, kt, vt = (torch.from_numpy(t[0, sl, h, :]) for t in (q, k, v))
            ro = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], scale=0.5)[0]
            rl = torch.logsumexp(0.5 * qt @ kt.T, dim=1)
            assert close(o[0, sl, h, :], ro.numpy()) and close(l[0, h, sl], rl.numpy())


def pin_unselected_keys_do_not_matter(fn):
    for c in CASES:
        q, k, v, sc, bm, blk, causal, mask, slopes = make_case(c)
        o1, l1 = call(fn, q, k, v, sc, bm, blk, causal, mask, slopes)
        B, S_q, H_q, _ = q.shape
        H_kv = k.shape[2]
        G = H_q // H_kv
        # For query block x of (b, h), change every key block it did not select.
        rng = np.random.default_rng(99)
        for b in range(B):
            for h in range(H_q):
                for x in range(bm.shape[2]):
                    k2, v2 = k.copy(), v.copy()
                    for y in range(bm.shape[3]):
                        if not bm[b, h, x, y]:
                            sl = slice(blk * y, blk * (y + 1))
                            k2[b, sl, h // G, :] += rnd(rng, *k2[b, sl, h // G, :].shape)
                            v2[b, sl, h // G, :] += rnd(rng, *v2[b, sl, h // G, :].shape)
                    o2, l2 = call(fn, q, k2, v2, sc, bm, blk, causal, mask, slopes)
                    rows = slice(blk * x, blk * (x + 1))
                    assert np.array_equal(o1[b, rows, h], o2[b, rows, h]), (c, b, h, x)
                    assert np.array_equal(l1[b, h, rows], l2[b, h, rows]), (c, b, h, x)


def pin_dense_and_empty(fn):
    for c in CASES:
        q, k, v, sc, bm, blk, causal, mask, slopes = make_case(c)
        ones = np.ones_like(bm)
        o, l = call(fn, q, k, v, sc, ones, blk, causal, mask, slopes)
        do, dl = oracle.attention(q, k, v, sc, causal=causal, key_padding_mask=mask, alibi_slopes=slopes)
        assert np.array_equal(o, do) and np.array_equal(l, dl), c
        zero = bm.copy()
        zero[:, :, 0, :] = 0
        o, l = call(fn, q, k, v, sc, zero, blk, causal, mask, slopes)
        assert (o[:, :blk] == 0).all() and np.isneginf(l[:, :, :blk]).all(), c


PINS = [pin_sdpa, pin_brute, pin_block_diagonal, pin_unselected_keys_do_not_matter, pin_dense_and_empty]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_sparse_oracle_pins(pin):
    pin(oracle.block_sparse_attention)


def test_shape_is_checked():
    q = np.zeros((1, 5, 2, 4))
    with pytest.raises(ValueError):
        oracle.block_sparse_attention(q, q, q, 1.0, np.ones((1, 2, 2, 3)), block=3)


# ------------------------------------------------------------- mutation test

def _patched(name, make):
    """The oracle with one module-level helper replaced (restored afterwards)."""
    def run(q, k, v, scale, bm, causal=False, key_padding_mask=None, alibi_slopes=None, block=128):
        saved = getattr(oatt, name)
        try:
            setattr(oatt, name, make(saved))
            return oatt.block_sparse_attention(q, k, v, scale, bm, causal=causal,
                                               key_padding_mask=key_padding_mask,
                                               alibi_slopes=alibi_slopes, block=block)
        finally:
            setattr(oatt, name, saved)
    return run


def _expand_with(index):
    """An expand_block_mask whose (row block, key block) lookup is replaced."""
    def make(_):
        def expand(bm_bh, S_q, S_k, rows=None, block=128):
            rows = np.arange(S_q) if rows is None else np.asarray(rows)
            bm = np.asarray(bm_bh) != 0
            return index(bm, rows, np.arange(S_k), block)
        return expand
    return make


def _safe_get(bm, a, b):
    return bm[np.clip(a, 0, bm.shape[0] - 1)][:, np.clip(b, 0, bm.shape[1] - 1)]


MUTANTS = {
    "block mask ignored": _patched("expand_block_mask", lambda f: (
        lambda bm, S_q, S_k, rows=None, block=128: np.ones(
            (S_q if rows is None else len(rows), S_k), dtype=bool))),
    "key block index off by one": _patched("expand_block_mask", _expand_with(
        lambda bm, rows, j, blk: _safe_get(bm, rows // blk, (j + 1) // blk))),
    "row block taken from the key axis offset": _patched("expand_block_mask", _expand_with(
        lambda bm, rows, j, blk: _safe_get(bm, (rows + 1) // blk, j // blk))),
    "block mask transposed": _patched("expand_block_mask", _expand_with(
        lambda bm, rows, j, blk: _safe_get(bm.T, rows // blk, j // blk))),
    "selection replaces the causal rule": _patched("visible", lambda f: (
        lambda S_q, S_k, causal, m=None, rows=None: f(S_q, S_k, False, m, rows))),
    "selection replaces the padding mask": _patched("visible", lambda f: (
        lambda S_q, S_k, causal, m=None, rows=None: f(S_q, S_k, causal, None, rows))),
}


def _rejects(pin, fn):
    try:
        pin(fn)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutants_run_and_differ(name):
    """Each planted mistake runs and changes the result on some pin case."""
    differs = False
    for c in CASES:
        args = make_case(c)
        o, l = call(MUTANTS[name], *args)
        ro, rl = call(oracle.block_sparse_attention, *args)
        differs = differs or not (np.array_equal(o, ro) and np.array_equal(l, rl))
    assert differs


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_reject_planted_mistakes(name):
    assert any(_rejects(p, MUTANTS[name]) for p in PINS), name
