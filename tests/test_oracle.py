"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin below checks ``oracle.attention`` (or, in the mutation test, a
deliberately broken copy of it) against one of:

* hand-derived values of the definition on toy inputs (tests/golden);
* closed forms: bottom-right causal averages, ALiBi geometric series;
* invariants the definition implies: single key, constant V, shift of all
  keys, GQA = repeated KV heads, padding = deleting keys, zero slopes, key
  permutation, split-and-merge of partial states;
* a library routine: torch's scaled_dot_product_attention and logsumexp in
  float64 on the CPU;
* an independent scalar brute force (``oracle.brute``) on tiny inputs.

The mutation test plants plausible mistakes in the oracle (on the CPU) and
checks that the pin suite rejects every one of them.
"""
import json
import math
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
import importlib

# The module itself: the package re-exports a function under the same name.
oatt = importlib.import_module("oracle.attention")
from workloads import WORKLOADS, Workload, alibi_slopes, make_inputs, to_f64

GOLDEN = Path(__file__).parent / "golden" / "worked_examples.json"


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def close(a, b, tol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape:
        return False
    inf = np.isinf(b)
    if not (np.isinf(a) == inf).all() or not (a[inf] == b[inf]).all():
        return False
    return bool(np.all(np.abs(a[~inf] - b[~inf]) <= tol * (1 + np.abs(b[~inf]))))


# ----------------------------------------------------------------- pin suite
# Each pin takes an attention implementation with the signature of
# oracle.attention and returns True when the implementation passes.

def pin_golden(attn):
    cases = json.loads(GOLDEN.read_text())["cases"]
    q = np.array([0.0, 1.0]).reshape(1, 2, 1, 1)
    kv = np.array([0.0, 1.0]).reshape(1, 2, 1, 1)
    for c in cases:
        mask = None if c["mask"] is None else np.array([c["mask"]], np.uint8)
        slopes = None if c["slope"] is None else np.array([c["slope"]])
        out, lse = attn(q, kv, kv, 1.0, c["causal"], mask, slopes)
        want_lse = np.array([float(x) for x in c["lse"]])
        if not close(out[0, :, 0, 0], np.array(c["out"])) or not close(lse[0, 0], want_lse):
            return False
    return True


def pin_causal_bottom_right(attn):
    """q = 0, v_j = j: row i averages keys 0..i+S_k-S_q (closed form)."""
    for S_q, S_k in ((5, 5), (3, 9), (6, 2)):
        q = np.zeros((1, S_q, 1, 2))
        k = np.ones((1, S_k, 1, 2))
        v = np.arange(S_k, dtype=np.float64).reshape(1, S_k, 1, 1)
        out, lse = attn(q, k, v, 0.7, True, None, None)
        for i in range(S_q):
            last = i + S_k - S_q
            if last < 0:
                ok = out[0, i, 0, 0] == 0 and lse[0, 0, i] == -np.inf
            else:
                ok = close(out[0, i, 0, 0], last / 2) and close(lse[0, 0, i], math.log(last + 1))
            if not ok:
                return False
    return True


def pin_alibi_geometric(attn):
    """q = 0: weights decay as r^|i - j| with r = e^-slope (geometric sums)."""
    slope, S = 0.3, 7
    r = math.exp(-slope)
    q = np.zeros((1, S, 1, 1))
    k = np.zeros((1, S, 1, 1))
    v = np.arange(S, dtype=np.float64).reshape(1, S, 1, 1)
    for causal in (True, False):
        out, lse = attn(q, k, v, 1.0, causal, None, np.array([slope]))
        for i in range(S):
            js = range(0, i + 1) if causal else range(S)
            wts = [r ** abs(i - j) for j in js]
            if not close(lse[0, 0, i], math.log(sum(wts))):
                return False
            if not close(out[0, i, 0, 0], sum(w * j for w, j in zip(wts, js)) / sum(wts)):
                return False
    # S_q < S_k: the bias is measured from the row's bottom-right position.
    q = np.zeros((1, 2, 1, 1))
    k = np.zeros((1, 5, 1, 1))
    v = np.arange(5, dtype=np.float64).reshape(1, 5, 1, 1)
    out, lse = attn(q, k, v, 1.0, True, None, np.array([slope]))
    for i in range(2):
        pos = i + 3
        wts = [r ** (pos - j) for j in range(pos + 1)]
        if not close(lse[0, 0, i], math.log(sum(wts))):
            return False
    return True


def pin_single_key(attn):
    rng = np.random.default_rng(1)
    q, k, v = rnd(rng, 2, 4, 3, 8), rnd(rng, 2, 1, 3, 8), rnd(rng, 2, 1, 3, 8)
    out, lse = attn(q, k, v, 0.4, False, None, None)
    want = np.einsum("bihd,bhd->bhi", q, k[:, 0]) * 0.4
    return bool((out == np.broadcast_to(v[:, :1], out.shape)).all()) and close(lse, want)


def pin_constant_v(attn):
    rng = np.random.default_rng(2)
    q, k = rnd(rng, 1, 9, 2, 4), rnd(rng, 1, 9, 2, 4)
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25, 3.0]), (1, 9, 2, 4)).copy()
    mask = np.ones((1, 9), np.uint8)
    mask[0, 6:] = 0
    out, _ = attn(q, k, v, 0.5, True, mask, np.array([0.2, 0.9]))
    return close(out, v, 1e-12)


def pin_shift_invariance(attn):
    """k_j -> k_j + u shifts every score of row i by scale q_i.u: out fixed, lse shifted."""
    rng = np.random.default_rng(3)
    q, k, v = rnd(rng, 1, 6, 2, 5), rnd(rng, 1, 8, 2, 5), rnd(rng, 1, 8, 2, 5)
    u = rnd(rng, 5)
    o1, l1 = attn(q, k, v, 0.3, False, None, None)
    o2, l2 = attn(q, k + u, v, 0.3, False, None, None)
    shift = 0.3 * np.einsum("bihd,d->bhi", q, u)
    return close(o1, o2, 1e-10) and close(l2, l1 + shift, 1e-10)


def pin_gqa_repeat(attn):
    rng = np.random.default_rng(4)
    q, k, v = rnd(rng, 2, 5, 6, 4), rnd(rng, 2, 7, 2, 4), rnd(rng, 2, 7, 2, 4)
    slopes = np.linspace(0.1, 0.6, 6)
    o1, l1 = attn(q, k, v, 0.5, True, None, slopes)
    o2, l2 = attn(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 0.5, True, None, slopes)
    return close(o1, o2) and close(l1, l2)


def pin_padding_is_deletion(attn):
    rng = np.random.default_rng(5)
    q, k, v = rnd(rng, 1, 4, 2, 3), rnd(rng, 1, 10, 2, 3), rnd(rng, 1, 10, 2, 3)
    keep = np.array([[1, 0, 1, 1, 0, 0, 1, 1, 1, 0]], np.uint8)
    o1, l1 = attn(q, k, v, 0.8, False, keep, None)
    idx = np.nonzero(keep[0])[0]
    o2, l2 = attn(q, k[:, idx], v[:, idx], 0.8, False, None, None)
    return close(o1, o2) and close(l1, l2)


def pin_zero_slopes(attn):
    rng = np.random.default_rng(6)
    q, k, v = rnd(rng, 1, 5, 3, 4), rnd(rng, 1, 5, 3, 4), rnd(rng, 1, 5, 3, 4)
    o1, l1 = attn(q, k, v, 0.5, True, None, np.zeros(3))
    o2, l2 = attn(q, k, v, 0.5, True, None, None)
    return close(o1, o2) and close(l1, l2)


def pin_key_permutation(attn):
    rng = np.random.default_rng(7)
    q, k, v = rnd(rng, 1, 4, 2, 3), rnd(rng, 1, 9, 2, 3), rnd(rng, 1, 9, 2, 3)
    perm = rng.permutation(9)
    o1, l1 = attn(q, k, v, 0.6, False, None, None)
    o2, l2 = attn(q, k[:, perm], v[:, perm], 0.6, False, None, None)
    return close(o1, o2) and close(l1, l2)


def pin_sdpa(attn):
    """torch SDPA (float64, CPU) with the bias and -inf for hidden keys as a float mask."""
    rng = np.random.default_rng(8)
    B, S_q, S_k, H, D = 2, 7, 11, 3, 5
    q, k, v = rnd(rng, B, S_q, H, D), rnd(rng, B, S_k, H, D), rnd(rng, B, S_k, H, D)
    mask = (rng.random((B, S_k)) > 0.3).astype(np.uint8)
    mask[:, -1] = 1
    slopes = np.array([0.5, 0.25, 0.125])
    scale = 0.45
    out, lse = attn(q, k, v, scale, True, mask, slopes)
    i_pos = np.arange(S_q)[:, None] + (S_k - S_q)
    j = np.arange(S_k)[None, :]
    fm = np.zeros((B, H, S_q, S_k))
    for h in range(H):
        fm[:, h] = -slopes[h] * np.abs(i_pos - j)
    hidden = (j > i_pos)[None, None] | (mask[:, None, None, :] == 0)
    fm = np.where(hidden, -np.inf, fm)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(fm), scale=scale)
    ref_lse = torch.logsumexp(scale * tq @ tk.transpose(-1, -2) + torch.from_numpy(fm), dim=-1)
    return close(out, ref.permute(0, 2, 1, 3).numpy(), 1e-10) and close(lse, ref_lse.numpy(), 1e-10)


def pin_brute(attn):
    rng = np.random.default_rng(9)
    for trial in range(12):
        B, S_q, S_k = 1 + trial % 2, 1 + trial % 5, 1 + (trial * 3) % 8
        H_kv = 1 + trial % 2
        H_q = H_kv * (1 + trial % 3)
        D = 1 + trial % 4
        causal = bool(trial % 2)
        q, k, v = rnd(rng, B, S_q, H_q, D), rnd(rng, B, S_k, H_kv, D), rnd(rng, B, S_k, H_kv, D)
        mask = (rng.random((B, S_k)) > 0.25).astype(np.uint8) if trial % 3 else None
        slopes = rng.random(H_q) if trial % 4 in (1, 2) else None
        scale = 0.2 + 0.1 * trial
        o1, l1 = attn(q, k, v, scale, causal, mask, slopes)
        o2, l2 = oracle.brute.attention(q.tolist(), k.tolist(), v.tolist(), scale, causal,
                                        None if mask is None else mask.tolist(),
                                        None if slopes is None else slopes.tolist())
        if not close(o1, np.array(o2)) or not close(l1, np.array(l2)):
            return False
    return True


def pin_split_merge(attn):
    """Merging per-split (out, lse) over any partition of the keys gives the unsplit result."""
    rng = np.random.default_rng(10)
    S = 23
    q, k, v = rnd(rng, 2, 1, 4, 6), rnd(rng, 2, S, 2, 6), rnd(rng, 2, S, 2, 6)
    mask = np.ones((2, S), np.uint8)
    mask[1, 5:12] = 0  # one split below is entirely hidden for batch row 1
    slopes = np.array([0.3, 0.1, 0.05, 0.7])
    full_o, full_l = attn(q, k, v, 0.5, False, mask, slopes)
    for bounds in ([0, S], [0, 12, S], [0, 5, 12, 13, S], [0, 1, 2, 3, 20, S]):
        parts = []
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            rngm = np.zeros((2, S), np.uint8)
            rngm[:, lo:hi] = 1
            parts.append(attn(q, k, v, 0.5, False, rngm & mask, slopes))
        # lse is [B, H, R]; the merge wants it aligned with out's [B, R, H].
        mo, ml = oracle.merge_states(np.stack([p[0] for p in parts]),
                                     np.stack([p[1].transpose(0, 2, 1) for p in parts]))
        if not close(mo, full_o, 1e-10) or not close(ml.transpose(0, 2, 1), full_l, 1e-10):
            return False
    return True


def pin_prob_rows_sum_to_one(attn):
    # Through the public signature: v = identity over keys returns P itself.
    rng = np.random.default_rng(11)
    S_k = 6
    q, k = rnd(rng, 1, 4, 1, S_k), rnd(rng, 1, S_k, 1, S_k)
    v = np.eye(S_k).reshape(1, S_k, 1, S_k)
    out, _ = attn(q, k, v, 0.9, True, None, np.array([0.4]))
    P = out[0, :, 0, :]
    return close(P.sum(axis=1), np.ones(4)) and bool((P >= 0).all())


PINS = [pin_golden, pin_causal_bottom_right, pin_alibi_geometric, pin_single_key, pin_constant_v,
        pin_shift_invariance, pin_gqa_repeat, pin_padding_is_deletion, pin_zero_slopes,
        pin_key_permutation, pin_sdpa, pin_brute, pin_split_merge, pin_prob_rows_sum_to_one]


def call_oracle(q, k, v, scale, causal, mask, slopes):
    return oracle.attention(q, k, v, scale, causal=causal, key_padding_mask=mask, alibi_slopes=slopes)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin):
    assert pin(call_oracle)


# ------------------------------------------------------------ other checks

@pytest.mark.parametrize("block", [1, 3, 64])
def test_online_recurrence_reaches_definition(block):
    """The pages' streaming recurrence (float64) equals the definition."""
    rng = np.random.default_rng(12)
    q, k, v = rnd(rng, 2, 70, 4, 8), rnd(rng, 2, 90, 2, 8), rnd(rng, 2, 90, 2, 8)
    mask = np.ones((2, 90), np.uint8)
    mask[0, 80:] = 0
    mask[1, :] = 0  # every row of batch 1 is fully hidden
    slopes = np.array([0.5, 0.2, 0.1, 0.05])
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, 0.35, causal, mask, slopes)
        o2, l2 = oracle.online_attention(q, k, v, 0.35, causal, mask, slopes, block=block)
        assert close(o1, o2, 1e-11) and close(l1, l2, 1e-11)


def test_prob_matrix_rows():
    """Rows of P sum to 1 over the visible keys and are 0 elsewhere.  P is read
    off ``attention`` itself: with one-hot value rows (v_j = e_j, S_k <= D)
    out[i, :S_k] is row i of P, so this pins the probabilities the outputs
    are built from, across GQA heads, ALiBi and padding."""
    rng = np.random.default_rng(13)
    B, S, H_q, H_kv, D = 2, 12, 4, 2, 16
    q, k = rnd(rng, B, S, H_q, D), rnd(rng, B, S, H_kv, D)
    v = np.zeros((B, S, H_kv, D))
    for j in range(S):
        v[:, j, :, j] = 1.0
    mask = np.ones((B, S), np.uint8)
    mask[1, 9:] = 0
    slopes = np.array([0.1, 0.3, 0.0, 0.7])
    out, lse = oracle.attention(q, k, v, 0.3, True, mask, slopes)
    for b in range(B):
        keep = np.tril(np.ones((S, S), bool)) & (mask[b] != 0)[None, :]
        for h in range(H_q):
            P = out[b, :, h, :S]
            assert np.abs(P.sum(axis=1) - 1).max() <= 1e-12
            assert (P[~keep] == 0).all() and (P[keep] > 0).all()
            assert (out[b, :, h, S:] == 0).all()
            # P[i, j] = exp(s[i, j] - lse[i]) for each visible key.
            hk = h // (H_q // H_kv)
            s = 0.3 * q[b, :, h] @ k[b, :, hk].T - slopes[h] * np.abs(np.arange(S)[:, None] - np.arange(S)[None, :])
            assert close(np.log(P[keep]), (s - lse[b, h][:, None])[keep], 1e-12)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(14)
    q, k, v = rnd(rng, 2, 40, 2, 4), rnd(rng, 2, 50, 2, 4), rnd(rng, 2, 50, 2, 4)
    rows = np.array([0, 3, 17, 39])
    o, l = oracle.attention(q, k, v, 0.5, True, None, np.array([0.2, 0.4]))
    os_, ls = oracle.attention(q, k, v, 0.5, True, None, np.array([0.2, 0.4]), rows=rows)
    assert close(os_, o[:, rows]) and close(ls, l[:, :, rows])


def test_overflow_inputs_stay_finite():
    """Scores far beyond the fp16 range: the float64 oracle stays finite and exact."""
    w = Workload("big", 1, 20, 20, 2, 2, 64, "fp16", causal=True, seed=3)
    inp = make_inputs(w, scale_qk=64.0)
    q, k = to_f64(inp.q), to_f64(inp.k)
    assert np.abs(np.einsum("bihd,bjhd->bhij", q, k)).max() > 65504
    o, l = oracle.attention(q, k, to_f64(inp.v), w.scale, causal=True)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    ob, lb = oracle.brute.attention(q.tolist(), k.tolist(), to_f64(inp.v).tolist(), w.scale, True)
    assert close(o, np.array(ob), 1e-12) and close(l, np.array(lb), 1e-12)


def test_generator_pins():
    """Seeded inputs reproduce the recorded first values and padding tails."""
    want = {
        "c1_fwd_256": [-1.525390625, -0.75, -0.65380859375, -1.609375],
        "c2_causal_pad16": [-1.041015625, 0.91650390625, -1.3037109375, -1.109375],
        "c3_causal_4096": [-0.07666015625, 0.35986328125, -0.7822265625, 0.071533203125],
        "c4_decode_32k": [-0.94140625, 1.263671875, -0.1837158203125, 0.1505126953125],
    }
    for name, vals in want.items():
        assert make_inputs(WORKLOADS[name]).q[0, 0, 0, :4].float().tolist() == vals
    s = alibi_slopes(32)
    assert s[0].item() == pytest.approx(2 ** -0.25) and s[31].item() == 2 ** -8


# ------------------------------------------------------------- mutation test

def _mutant(patches):
    """An oracle with some module-level helpers replaced (restored afterwards)."""
    def run(q, k, v, scale, causal, mask, slopes):
        saved = {n: getattr(oatt, n) for n in patches}
        try:
            for n, f in patches.items():
                setattr(oatt, n, f(saved[n]))
            return call_oracle(q, k, v, scale, causal, mask, slopes)
        finally:
            for n, f in saved.items():
                setattr(oatt, n, f)
    return run


def _wrap_attention(transform):
    def run(q, k, v, scale, causal, mask, slopes):
        return transform(q, k, v, scale, causal, mask, slopes)
    return run


MUTANTS = {
    "bias sign flipped": _mutant({"alibi_bias": lambda f: (lambda s, a, b, rows=None: -f(s, a, b, rows))}),
    "bias without abs": _mutant({"alibi_bias": lambda f: (
        lambda s, S_q, S_k, rows=None: -float(s) * (
            (np.arange(S_q) if rows is None else np.asarray(rows))[:, None] + (S_k - S_q)
            - np.arange(S_k)[None, :]).astype(float))}),
    "causal top-left": _mutant({"visible": lambda f: (
        lambda S_q, S_k, causal, m=None, rows=None: f(S_q, S_k, causal, m, rows)
        & ((np.arange(S_k)[None, :] <= (np.arange(S_q) if rows is None else np.asarray(rows))[:, None])
           | (not causal)))}),
    "mask polarity inverted": _mutant({"visible": lambda f: (
        lambda S_q, S_k, causal, m=None, rows=None: f(S_q, S_k, causal, None if m is None else (np.asarray(m) == 0), rows))}),
    "softmax lse drops the max": _mutant({"_softmax_rows": lambda f: (
        lambda s: (f(s)[0], f(s)[1] - np.where(np.isfinite(s.max(axis=1)), s.max(axis=1), 0.0)))}),
    "scale ignored": _wrap_attention(lambda q, k, v, sc, c, m, sl: call_oracle(q, k, v, 1.0, c, m, sl)),
    "GQA heads interleaved": _wrap_attention(
        lambda q, k, v, sc, c, m, sl: call_oracle(
            q, np.repeat(k, q.shape[2] // k.shape[2], axis=2)[:, :, _interleave(q.shape[2], k.shape[2])],
            np.repeat(v, q.shape[2] // v.shape[2], axis=2)[:, :, _interleave(q.shape[2], v.shape[2])],
            sc, c, m, sl)),
    "key/value rows misaligned": _wrap_attention(
        lambda q, k, v, sc, c, m, sl: call_oracle(q, k, np.roll(v, 1, axis=1), sc, c, m, sl)),
}


def _interleave(H_q, H_kv):
    """Head order that maps query head h to KV head h % H_kv instead of h // G."""
    G = H_q // H_kv
    return np.array([(h % H_kv) * G for h in range(H_q)])


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutants_run_and_differ(name):
    """Each planted mistake runs and changes the result on a generic input
    (so that its rejection below is not an artefact of the test machinery)."""
    rng = np.random.default_rng(77)
    q, k, v = rnd(rng, 2, 6, 4, 3), rnd(rng, 2, 8, 2, 3), rnd(rng, 2, 8, 2, 3)
    mask = np.ones((2, 8), np.uint8)
    mask[0, 5] = 0
    differs = False
    for causal in (True, False):   # some mistakes only show without the causal rule
        args = (q, k, v, 0.7, causal, mask, np.array([0.5, 0.25, 0.125, 0.0625]))
        got = MUTANTS[name](*args)
        ref = call_oracle(*args)
        differs = differs or not (close(got[0], ref[0], 1e-9) and close(got[1], ref[1], 1e-9))
    assert differs


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_reject_planted_mistakes(name):
    failed = [p.__name__ for p in PINS if not _safe(p, MUTANTS[name])]
    assert failed, f"no pin catches the planted mistake: {name}"


def _safe(pin, impl):
    try:
        return pin(impl)
    except Exception:
        return False
