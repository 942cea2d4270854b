"""Pins of the additive-mask / dropout oracle (``oracle.attention_ext``) and
of its Philox4x32-10 generator (``oracle.philox``).

Checked against facts outside the oracle's own code path:

* the generator: the known-answer vectors published with the Random123
  library of Salmon et al. for philox4x32 with 10 rounds (counter and key all
  zeros; all ones; the hexadecimal digits of pi), and the vectorised version
  against the scalar one;
* the additive mask: torch's scaled_dot_product_attention in float64 with the
  bias (plus ALiBi, plus -inf where the causal rule or the padding hides a
  key) as its float attn_mask, for bias shapes that broadcast over batch or
  heads; a -inf bias equals the boolean mask;
* dropout: the scalar brute force of ``oracle.brute`` (one generator call
  per element); the kept fraction and the mean output over many seeds
  (statistics of a Bernoulli(1 - p) mask with 1 / (1 - p) scaling, whose
  mean is the undropped output); lse does not change with dropout; p = 0 is
  the plain definition.

A mutation test plants plausible mistakes (on the CPU) and checks that the
pins reject each.
"""
import importlib

import numpy as np
import pytest
import torch

import oracle
from oracle import brute, philox

oatt = importlib.import_module("oracle.attention")

# Known-answer vectors of philox4x32-10 (Random123 "kat_vectors").
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def close(a, b, tol=1e-10):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape:
        return False
    fin = np.isfinite(b)
    return bool(np.array_equal(np.isfinite(a), fin) and np.all(a[~fin] == b[~fin])
                and np.all(np.abs(a[fin] - b[fin]) <= tol * (1 + np.abs(b[fin]))))


def make(seed, B=2, S_q=6, S_k=9, H_q=4, H_kv=2, D=4, bias_shape="bhqk", causal=True, mask=True,
         alibi=True, ninf=True):
    rng = np.random.default_rng(seed)
    q, k, v = rnd(rng, B, S_q, H_q, D), rnd(rng, B, S_k, H_kv, D), rnd(rng, B, S_k, H_kv, D)
    shapes = {"bhqk": (B, H_q, S_q, S_k), "b1qk": (B, 1, S_q, S_k), "qk": (S_q, S_k), "b11k": (B, 1, 1, S_k)}
    bias = rnd(rng, *shapes[bias_shape])
    if ninf:
        bias[bias > 1.2] = -np.inf
    m = None
    if mask:
        m = np.ones((B, S_k), np.uint8)
        m[:, -1] = 0
        m[0, 2] = 0
    sl = rng.uniform(0.1, 0.9, H_q) if alibi else None
    return q, k, v, 0.7, causal, m, sl, bias


def sdpa_ref(q, k, v, scale, causal, mask, slopes, bias):
    B, S_q, H_q, D = q.shape
    S_k, H_kv = k.shape[1], k.shape[2]
    G = H_q // H_kv
    ab = np.broadcast_to(bias, (B, H_q, S_q, S_k))
    out = np.zeros((B, S_q, H_q, D))
    lse = np.full((B, H_q, S_q), -np.inf)
    for b in range(B):
        for h in range(H_q):
            am = torch.from_numpy(ab[b, h].copy())
            i = torch.arange(S_q, dtype=torch.float64)[:, None] + (S_k - S_q)
            j = torch.arange(S_k, dtype=torch.float64)[None, :]
            if slopes is not None:
                am = am - float(slopes[h]) * (i - j).abs()
            if causal:
                am = torch.where(j > i, torch.tensor(float("-inf"), dtype=torch.float64), am)
            if mask is not None:
                am = torch.where(torch.from_numpy(mask[b] == 0)[None, :],
                                 torch.tensor(float("-inf"), dtype=torch.float64), am)
            qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(t)) for t in
                          (q[b, :, h], k[b, :, h // G], v[b, :, h // G]))
            rows = torch.isfinite(am).any(dim=1)
            if rows.any():
                o = torch.nn.functional.scaled_dot_product_attention(
                    qt[rows][None], kt[None], vt[None], attn_mask=am[rows][None], scale=float(scale))[0]
                out[b, rows.numpy(), h] = o.numpy()
                lse[b, h, rows.numpy()] = torch.logsumexp(float(scale) * qt[rows] @ kt.T + am[rows], dim=1).numpy()
    return out, lse


# ------------------------------------------------------------------ pins

def pin_philox_kat(gen):
    for ctr, key, want in KAT:
        assert tuple(gen.philox4x32_10(ctr, key)) == want


def pin_philox_vectorised(gen):
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2 ** 32, (4, 300), dtype=np.uint64)
    key = (0x1234ABCD, 0x0F0E0D0C)
    words = gen.philox_words(*c, *key)
    for n in range(300):
        assert tuple(int(w[n]) for w in words) == philox.philox4x32_10(tuple(int(x[n]) for x in c), key)
    for ctr, key, want in KAT:
        assert tuple(int(w) for w in gen.philox_words(*ctr, *key)) == want


def pin_bias_sdpa(fn):
    for n, shape in enumerate(["bhqk", "b1qk", "qk", "b11k"]):
        for causal in (False, True):
            q, k, v, sc, c, m, sl, bias = make(10 + n, bias_shape=shape, causal=causal)
            o, l = fn(q, k, v, sc, c, m, sl, attn_bias=bias)
            ro, rl = sdpa_ref(q, k, v, sc, c, m, sl, bias)
            assert close(o, ro) and close(l, rl), (shape, causal)


def pin_ninf_bias_is_mask(fn):
    q, k, v, sc, c, m, sl, _ = make(20, mask=False)
    m = np.ones((2, 9), np.uint8)
    m[0, [1, 4]] = 0
    m[1, 8] = 0
    bias = np.where(m[:, None, None, :] == 0, -np.inf, 0.0)
    o, l = fn(q, k, v, sc, c, None, sl, attn_bias=bias)
    ro, rl = oracle.attention(q, k, v, sc, causal=c, key_padding_mask=m, alibi_slopes=sl)
    assert close(o, ro, 1e-12) and close(l, rl, 1e-12)


def pin_plain_without_extras(fn):
    q, k, v, sc, c, m, sl, _ = make(21)
    o, l = fn(q, k, v, sc, c, m, sl)
    ro, rl = oracle.attention(q, k, v, sc, causal=c, key_padding_mask=m, alibi_slopes=sl)
    assert close(o, ro, 1e-12) and close(l, rl, 1e-12)


def pin_brute_dropout(fn):
    # The last case spans three 64-key windows: both halves of the words and
    # several block counters per row.
    for n, (p, seed, offset, S_k) in enumerate([(0.3, 1234567, 0, 10), (0.5, 2 ** 40 + 99, 7, 10),
                                                 (0.1, 3, 1, 10), (0.4, 2 ** 63 + 5, 3, 150)]):
        q, k, v, sc, c, m, sl, bias = make(30 + n, B=2, S_q=5 if S_k < 64 else 2, S_k=S_k, H_q=2, H_kv=1, D=3)
        S_q = q.shape[1]
        o, l = fn(q, k, v, sc, c, m, sl, attn_bias=bias, dropout_p=p, seed=seed, offset=offset)
        bo, bl = brute.attention(q.tolist(), k.tolist(), v.tolist(), sc, c, m.tolist(), sl.tolist(),
                                 attn_bias=np.broadcast_to(bias, (2, 2, S_q, S_k)).tolist(),
                                 dropout_p=p, seed=seed, offset=offset)
        assert close(o, np.array(bo)) and close(l, np.array(bl)), (p, seed)


def pin_dropout_uses_each_half_once(fn):
    """Over whole 64-key windows a row's decisions use every 16-bit half of
    the row's blocks exactly once: the values of keys 0 .. 191 are, as a
    multiset, the 24 blocks' 192 halves (computed here block by block)."""
    seed, offset, H_q, b, h = 0x0123456789ABCDEF, 9, 3, 1, 2
    for row in (0, 5):
        vals = philox.dropout_values(b, h, H_q, [row], 192, seed, offset)[0]
        halves = []
        for c0 in range(24):
            for w in philox.philox4x32_10((c0, row, b * H_q + h, offset), (seed & 0xFFFFFFFF, seed >> 32)):
                halves += [w & 0xFFFF, w >> 16]
        assert sorted(int(x) for x in vals) == sorted(halves)


def pin_dropout_statistics(fn):
    """Kept fraction ~ 1 - p, the mean over seeds ~ the undropped output, lse unchanged."""
    rng = np.random.default_rng(40)
    B, S, H, D, p = 1, 64, 2, 4, 0.25
    q, k, v = rnd(rng, B, S, H, D) * 0.3, rnd(rng, B, S, H, D) * 0.3, rnd(rng, B, S, H, D)
    base_o, base_l = fn(q, k, v, 0.5, False, None, None)
    seeds = 400
    acc = np.zeros_like(base_o)
    for s in range(seeds):
        o, l = fn(q, k, v, 0.5, False, None, None, dropout_p=p, seed=1000 + s)
        assert close(l, base_l, 1e-12)
        acc += o
    mean = acc / seeds
    # Each output is a sum of ~64 terms of size ~1/64 with Bernoulli(1-p) / (1-p) weights:
    # the standard error of the mean over seeds is about sqrt(p/(1-p)/64/seeds) ~ 0.0036.
    assert np.abs(mean - base_o).max() < 0.025
    keep = philox.keep_mask(0, 1, H, np.arange(S), 4096, p, 77)
    frac = keep.mean()
    n = keep.size
    assert abs(frac - (1 - p)) < 5 * np.sqrt(p * (1 - p) / n)


PINS = [pin_bias_sdpa, pin_ninf_bias_is_mask, pin_plain_without_extras, pin_brute_dropout,
        pin_dropout_statistics, pin_dropout_uses_each_half_once]
GEN_PINS = [pin_philox_kat, pin_philox_vectorised]


def call_ext(q, k, v, sc, c, m, sl, **kw):
    return oracle.attention_ext(q, k, v, sc, causal=c, key_padding_mask=m, alibi_slopes=sl, **kw)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_ext_oracle_pins(pin):
    pin(call_ext)


@pytest.mark.parametrize("pin", GEN_PINS, ids=lambda p: p.__name__)
def test_philox_pins(pin):
    pin(philox)


def test_threshold_and_validation():
    assert philox.drop_threshold(0.0) == 0
    assert philox.drop_threshold(0.5) == 2 ** 15
    assert philox.drop_threshold(0.1) == 6553
    assert philox.drop_threshold(1 - 2 ** -40) == 2 ** 16 - 1
    for bad in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            philox.drop_threshold(bad)


# ------------------------------------------------------------- mutation test

class _Patched:
    """An oracle with one attribute of a module replaced while it runs."""
    def __init__(self, mod, name, make):
        self.mod, self.name, self.make = mod, name, make

    def __call__(self, *a, **kw):
        saved = getattr(self.mod, self.name)
        try:
            setattr(self.mod, self.name, self.make(saved))
            return call_ext(*a, **kw)
        finally:
            setattr(self.mod, self.name, saved)


def _swapped_keep(b, h, H_q, rows, S_k, p, seed, offset=0):
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(S_k, dtype=np.int64)
    words = philox.philox_words(rows[:, None] // 4, j[None, :], b * H_q + h, offset,
                                seed & 0xFFFFFFFF, seed >> 32)
    w = np.choose((rows % 4)[:, None].repeat(S_k, axis=1), words) & np.uint64(0xFFFF)
    return w >= np.uint64(philox.drop_threshold(p))


def _halves_swapped(b, h, H_q, rows, S_k, p, seed, offset=0):
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(S_k, dtype=np.int64)
    c0, word, half = philox.decision_slot(j)
    words = philox.philox_words(c0[None, :], rows[:, None], b * H_q + h, offset,
                                seed & 0xFFFFFFFF, seed >> 32)
    w = np.choose(word[None, :].repeat(len(rows), axis=0), words)
    v = (w >> (np.uint64(16) * (1 - half).astype(np.uint64))[None, :]) & np.uint64(0xFFFF)
    return v >= np.uint64(philox.drop_threshold(p))


def _wrap(transform):
    def run(q, k, v, sc, c, m, sl, **kw):
        return transform(q, k, v, sc, c, m, sl, **kw)
    return run


MUTANTS = {
    "dropout not rescaled": _Patched(philox, "keep_mask", lambda f: (
        lambda b, h, H, rows, S_k, p, seed, offset=0: f(b, h, H, rows, S_k, p, seed, offset) * (1 - p))),
    "dropout keeps the words below the threshold": _Patched(philox, "keep_mask", lambda f: (
        lambda b, h, H, rows, S_k, p, seed, offset=0: ~f(b, h, H, rows, S_k, p, seed, offset))),
    "dropout counter with row and key swapped": _Patched(philox, "keep_mask", lambda f: _swapped_keep),
    "dropout word halves swapped": _Patched(philox, "keep_mask", lambda f: _halves_swapped),
    "bias sign flipped": _wrap(lambda q, k, v, sc, c, m, sl, **kw: call_ext(
        q, k, v, sc, c, m, sl, **{**kw, "attn_bias": None if kw.get("attn_bias") is None else -kw["attn_bias"]})),
    "bias added before the scale": _wrap(lambda q, k, v, sc, c, m, sl, **kw: call_ext(
        q, k, v, sc, c, m, sl, **{**kw, "attn_bias": None if kw.get("attn_bias") is None else sc * kw["attn_bias"]})),
    "bias ignored": _wrap(lambda q, k, v, sc, c, m, sl, **kw: call_ext(
        q, k, v, sc, c, m, sl, **{**kw, "attn_bias": None})),
}
GEN_MUTANTS = {
    "philox one round short": lambda: _gen_with(ROUNDS=9),
    "philox multipliers swapped": lambda: _gen_with(M0=philox.M1, M1=philox.M0),
}


def _gen_with(**attrs):
    saved = {n: getattr(philox, n) for n in attrs}
    for n, val in attrs.items():
        setattr(philox, n, val)
    return saved


def _rejects(pin, fn):
    try:
        pin(fn)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutants_differ_and_are_rejected(name):
    q, k, v, sc, c, m, sl, bias = make(50)
    a = MUTANTS[name](q, k, v, sc, c, m, sl, attn_bias=bias, dropout_p=0.3, seed=5)
    b = call_ext(q, k, v, sc, c, m, sl, attn_bias=bias, dropout_p=0.3, seed=5)
    assert not (np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])), "mutant changes nothing"
    assert any(_rejects(p, MUTANTS[name]) for p in PINS), name


@pytest.mark.parametrize("name", list(GEN_MUTANTS))
def test_generator_mutants_are_rejected(name):
    saved = GEN_MUTANTS[name]()
    try:
        assert any(_rejects(p, philox) for p in GEN_PINS), name
    finally:
        for n, val in saved.items():
            setattr(philox, n, val)
