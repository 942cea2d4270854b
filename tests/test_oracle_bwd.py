"""Pins of the float64 backward oracle (``oracle.attention_bwd``).

The gradients are checked against facts that do not come from the oracle's
own formula:

* torch autograd in float64 on the CPU, through an independently written
  forward (scores, bias, -inf for hidden keys, softmax, product with V; GQA by
  repeating the key/value heads, whose gradients autograd then sums);
* central finite differences of the forward oracle (itself pinned in
  test_oracle.py) on tiny inputs;
* closed forms: constant value rows give dq = dk = 0; a row with no visible
  key and a key hidden from every row get zero gradients.

A mutation test plants plausible mistakes in the oracle's per-head gradient
step (on the CPU) and checks that the pins reject each of them.
"""
import numpy as np
import pytest
import torch

import oracle
import importlib

# The module itself: the package re-exports a function under the same name.
oatt = importlib.import_module("oracle.attention")


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def close(a, b, tol):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return a.shape == b.shape and bool(np.all(np.abs(a - b) <= tol * (1 + np.abs(b))))


def autograd_ref(q, k, v, dout, scale, causal, mask, slopes):
    """float64 torch autograd of an independently written forward."""
    B, S_q, H_q, D = q.shape
    S_k, H_kv = k.shape[1], k.shape[2]
    G = H_q // H_kv
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    kk = tk.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)   # [B, H_q, S_k, D]
    vv = tv.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    qq = tq.permute(0, 2, 1, 3)
    s = scale * qq @ kk.transpose(-1, -2)                       # [B, H_q, S_q, S_k]
    i_pos = torch.arange(S_q)[:, None] + (S_k - S_q)
    j = torch.arange(S_k)[None, :]
    if slopes is not None:
        s = s - torch.tensor(slopes)[None, :, None, None] * (i_pos - j).abs()
    hidden = torch.zeros(B, 1, S_q, S_k, dtype=torch.bool)
    if causal:
        hidden = hidden | (j > i_pos)
    if mask is not None:
        hidden = hidden | (torch.tensor(mask) == 0)[:, None, None, :]
    s = s.masked_fill(hidden, float("-inf"))
    out = torch.softmax(s, dim=-1) @ vv                         # [B, H_q, S_q, D]
    (out.permute(0, 2, 1, 3) * torch.tensor(dout)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


# ----------------------------------------------------------------- pin suite
# Each pin takes a backward implementation with the signature of
# oracle.attention_bwd and returns True when it passes.

def pin_autograd(bwd):
    rng = np.random.default_rng(31)
    ok = True
    for (B, S_q, S_k, H_q, H_kv, D, causal, use_mask, use_alibi) in [
            (2, 6, 9, 4, 2, 5, True, True, True),
            (1, 7, 7, 3, 3, 4, False, False, False),
            (2, 5, 5, 2, 1, 3, True, False, True)]:
        q, k, v = rnd(rng, B, S_q, H_q, D), rnd(rng, B, S_k, H_kv, D), rnd(rng, B, S_k, H_kv, D)
        dout = rnd(rng, B, S_q, H_q, D)
        mask = None
        if use_mask:
            mask = (rng.random((B, S_k)) > 0.35).astype(np.uint8)
            mask[:, 0] = 1  # every row keeps a visible key (softmax of an all -inf row is NaN)
        slopes = 0.5 ** np.arange(1, H_q + 1) if use_alibi else None
        got = bwd(q, k, v, dout, 0.4, causal, mask, slopes)
        ref = autograd_ref(q, k, v, dout, 0.4, causal, mask, slopes)
        ok = ok and all(close(g, r, 1e-10) for g, r in zip(got, ref))
    return ok


def pin_finite_differences(bwd):
    """Central differences of sum(out * dout) through the forward oracle."""
    rng = np.random.default_rng(32)
    B, S_q, S_k, H_q, H_kv, D = 1, 3, 4, 2, 1, 3
    q, k, v = rnd(rng, B, S_q, H_q, D), rnd(rng, B, S_k, H_kv, D), rnd(rng, B, S_k, H_kv, D)
    dout = rnd(rng, B, S_q, H_q, D)
    mask = np.array([[1, 1, 0, 1]], np.uint8)
    slopes = np.array([0.3, 0.7])
    scale, causal = 0.6, True
    got = bwd(q, k, v, dout, scale, causal, mask, slopes)

    def f(q_, k_, v_):
        out, _ = oracle.attention(q_, k_, v_, scale, causal, mask, slopes)
        return float((out * dout).sum())

    eps = 1e-6
    grads = []
    for which, x in enumerate((q, k, v)):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            g[idx] = (f(*args_p) - f(*args_m)) / (2 * eps)
        grads.append(g)
    return all(np.abs(a - b).max() <= 1e-7 for a, b in zip(got, grads))


def pin_constant_values(bwd):
    """With every value row equal, the output is that row whatever the
    probabilities, so q and k get no gradient."""
    rng = np.random.default_rng(33)
    B, S_q, S_k, H_q, H_kv, D = 2, 5, 7, 4, 2, 6
    q, k = rnd(rng, B, S_q, H_q, D), rnd(rng, B, S_k, H_kv, D)
    v = np.broadcast_to(rnd(rng, 1, 1, H_kv, D), (B, S_k, H_kv, D)).copy()
    dout = rnd(rng, B, S_q, H_q, D)
    dq, dk, dv = bwd(q, k, v, dout, 0.5, True, None, 0.25 ** np.arange(1, H_q + 1))
    return np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12 and np.abs(dv).max() > 1e-3


def pin_hidden_rows_and_keys(bwd):
    """A row with no visible key and a key hidden from every row get zero
    gradients; a row with a single visible key gets dq = 0 (its softmax is
    the constant 1); rows with several visible keys and visible keys do
    not."""
    rng = np.random.default_rng(34)
    B, S_q, S_k, H, D = 1, 6, 4, 2, 3   # causal with S_q > S_k: rows 0, 1 see nothing
    q, k, v = rnd(rng, B, S_q, H, D), rnd(rng, B, S_k, H, D), rnd(rng, B, S_k, H, D)
    dout = rnd(rng, B, S_q, H, D)
    mask = np.array([[1, 0, 1, 1]], np.uint8)  # key 1 hidden from every row
    dq, dk, dv = bwd(q, k, v, dout, 0.7, True, mask, None)
    # Visible keys: row i sees j <= i - 2 except key 1, so rows 0-1 see none,
    # rows 2-3 only key 0, rows 4-5 two or three keys.
    return (np.abs(dq[:, :2]).max() == 0 and np.abs(dk[:, 1]).max() == 0
            and np.abs(dv[:, 1]).max() == 0 and np.abs(dq[:, 2:4]).max() < 1e-15
            and np.abs(dq[:, 4:]).min() > 0 and np.abs(dv[:, 0]).min() > 0)


PINS = [pin_autograd, pin_finite_differences, pin_constant_values, pin_hidden_rows_and_keys]


def call_bwd(q, k, v, dout, scale, causal, mask, slopes):
    return oracle.attention_bwd(q, k, v, dout, scale, causal=causal, key_padding_mask=mask,
                                alibi_slopes=slopes)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_bwd_oracle_pins(pin):
    assert pin(call_bwd)


# ------------------------------------------------------------- mutation test

def _head_mutant(fn):
    """The oracle with its per-head gradient step replaced."""
    def run(*args):
        saved = oatt._bwd_head
        try:
            oatt._bwd_head = fn
            return call_bwd(*args)
        finally:
            oatt._bwd_head = saved
    return run


def _no_row_dot(P, do, qh, kh, vh, scale):
    dP = do @ vh.T
    dS = P * dP
    return scale * (dS @ kh), scale * (dS.T @ qh), P.T @ do


def _unweighted_row_dot(P, do, qh, kh, vh, scale):
    dP = do @ vh.T
    dS = P * (dP - dP.mean(axis=1)[:, None])
    return scale * (dS @ kh), scale * (dS.T @ qh), P.T @ do


def _dk_unscaled(P, do, qh, kh, vh, scale):
    dq, dk, dv = oatt.__dict__["_bwd_head_orig"](P, do, qh, kh, vh, scale)
    return dq, dk / scale, dv


def _dv_from_dS(P, do, qh, kh, vh, scale):
    dP = do @ vh.T
    dS = P * (dP - (P * dP).sum(axis=1)[:, None])
    return scale * (dS @ kh), scale * (dS.T @ qh), dS.T @ do


def _gqa_first_head_only(q, k, v, dout, scale, causal, mask, slopes):
    """Key/value gradients taken from one query head of each group, not summed."""
    G = q.shape[2] // k.shape[2]
    rk = np.repeat(k, G, axis=2)
    rv = np.repeat(v, G, axis=2)
    dq, dk, dv = call_bwd(q, rk, rv, dout, scale, causal, mask, slopes)
    return dq, dk[:, :, ::G], dv[:, :, ::G]


oatt._bwd_head_orig = oatt._bwd_head
MUTANTS = {
    "row dot omitted": _head_mutant(_no_row_dot),
    "row dot not weighted by P": _head_mutant(_unweighted_row_dot),
    "dk missing the scale": _head_mutant(_dk_unscaled),
    "dv from dS instead of P": _head_mutant(_dv_from_dS),
    "GQA gradients not summed": _gqa_first_head_only,
}


def _safe(pin, impl):
    try:
        return pin(impl)
    except Exception:
        return False


@pytest.mark.parametrize("name", list(MUTANTS))
def test_bwd_mutants_run_and_differ(name):
    """Each planted mistake runs and changes the gradients on a generic input
    (so that its rejection below is not an artefact of the test machinery)."""
    rng = np.random.default_rng(78)
    args = (rnd(rng, 2, 6, 4, 3), rnd(rng, 2, 8, 2, 3), rnd(rng, 2, 8, 2, 3), rnd(rng, 2, 6, 4, 3),
            0.7, True, None, np.array([0.5, 0.25, 0.125, 0.0625]))
    got = MUTANTS[name](*args)
    ref = call_bwd(*args)
    assert not all(close(g, r, 1e-9) for g, r in zip(got, ref))


@pytest.mark.parametrize("name", list(MUTANTS))
def test_bwd_pins_reject_planted_mistakes(name):
    failed = [p.__name__ for p in PINS if not _safe(p, MUTANTS[name])]
    assert failed, f"no pin catches the planted mistake: {name}"


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def test_grad_rounding_term_bounds_operand_rounding():
    """The GPU tests' gradient rounding term (``parity.grad_rounding``): its
    dv part is u times the oracle's dv of |dout|, and a float64 backward whose
    dS and P are rounded to bfloat16 before the second products stays within
    it element by element."""
    from parity import grad_rounding
    from workloads import Workload, make_dout, make_inputs, to_f64
    w = Workload("grad_term", 2, 40, 56, 8, 2, 16, "bf16", causal=True, alibi=True, random_tail=12, seed=79)
    inp = make_inputs(w)
    do = to_f64(make_dout(w))
    q, k, v = to_f64(inp.q), to_f64(inp.k), to_f64(inp.v)
    mask, sl = inp.mask.numpy(), inp.slopes.numpy()
    eq, ek, ev = grad_rounding(inp, do, torch.bfloat16)
    u = 2.0 ** -8
    dv_abs = oracle.attention_bwd(q, k, v, np.abs(do), w.scale, causal=True, key_padding_mask=mask,
                                  alibi_slopes=sl)[2]
    assert np.allclose(ev, u * dv_abs, rtol=1e-12, atol=0)
    ref = oracle.attention_bwd(q, k, v, do, w.scale, causal=True, key_padding_mask=mask, alibi_slopes=sl)
    G = w.H_q // w.H_kv
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(w.B):
        keep = oracle.visible(w.S_q, w.S_k, True, mask[b])
        for h in range(w.H_q):
            hk = h // G
            P, _ = oatt._softmax_rows(oatt._scores(q[b, :, h], k[b, :, hk], w.scale, keep,
                                                   oracle.alibi_bias(float(sl[h]), w.S_q, w.S_k)))
            dP = do[b, :, h] @ v[b, :, hk].T
            dS = _bf16(P * (dP - (P * dP).sum(axis=1, keepdims=True)))
            dq[b, :, h] = w.scale * (dS @ k[b, :, hk])
            dk[b, :, hk] += w.scale * (dS.T @ q[b, :, h])
            dv[b, :, hk] += _bf16(P).T @ do[b, :, h]
    for g, r, e in zip((dq, dk, dv), ref, (eq, ek, ev)):
        err = np.abs(g - r)
        assert (err <= e * (1 + 1e-9) + 1e-12).all()
        assert err.max() > 0.1 * e.max()      # the term is not vacuous at this size
