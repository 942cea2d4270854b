"""Float64 CPU oracle for exact attention with online-softmax semantics.

Test infrastructure only (see the package docstring): the HIP library never
imports this module and this module never imports the library.

What is computed, and where the pages define it
-----------------------------------------------
For batch b, query head h (reading key/value head ``h // (H_q / H_kv)``, the
consecutive grouping of the "Attention API" page, ``compute_hybrid_attention_store``,
where queries are viewed as ``(T, H_kv, G, D)``), query row i and key j:

* score ``s[i, j] = scale * <q_i, k_j> + bias[i, j]`` — the scaled product of
  "StreamAttention: Fused Online Softmax Attention", section "Kernel Design",
  with the ALiBi bias of its "API Reference" (``alibi_slopes``);
* a key is visible to a row when it passes the causal rule and the boolean
  key-padding mask (nonzero = keep; the "Quick Start" builds the mask as ones
  and clears the positions to hide);
* ``lse[i] = log(sum over visible j of exp(s[i, j]))`` (the log-sum-exp that
  section "Kernel Design" returns next to the output) and
  ``out[i] = sum over visible j of exp(s[i, j] - lse[i]) * v_j``.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):

* causal alignment is bottom-right: key j is visible to row i when
  ``j <= i + S_k - S_q`` (the same as ``j <= i`` when ``S_q == S_k``);
* the ALiBi bias is ``-slope_h * |i + S_k - S_q - j|`` added after scaling;
* a row with no visible key gives ``out = 0`` and ``lse = -inf`` (the
  fully-masked-row guard of the "flash-attn-volta" page, section "Stability",
  and the zero output for an empty cache of the "Attention API" page,
  ``compute_hybrid_attention``);
* the log is natural.

Arithmetic is float64 throughout; inputs are upcast from whatever values the
caller passes (the exact fp16/bf16 values the GPU receives, and the float32
``scale`` and slopes that cross the C ABI).
"""
from __future__ import annotations

import numpy as np

from . import philox


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def visible(S_q, S_k, causal, mask_row=None, rows=None):
    """Boolean ``[R, S_k]`` visibility of keys to query rows.

    ``rows`` selects query row indices (default all ``S_q``); ``mask_row`` is
    the batch row of the key-padding mask, nonzero meaning keep.
    """
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    i_abs = rows + (S_k - S_q)
    j = np.arange(S_k)
    keep = np.ones((len(rows), S_k), dtype=bool)
    if causal:
        keep &= j[None, :] <= i_abs[:, None]
    if mask_row is not None:
        keep &= (np.asarray(mask_row) != 0)[None, :]
    return keep


def alibi_bias(slope, S_q, S_k, rows=None):
    """``[R, S_k]`` additive bias ``-slope * |i + S_k - S_q - j|`` in float64."""
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    i_abs = (rows + (S_k - S_q)).astype(np.float64)
    j = np.arange(S_k, dtype=np.float64)
    return -float(slope) * np.abs(i_abs[:, None] - j[None, :])


def _scores(qbh, kbh, scale, keep, bias):
    s = float(scale) * (qbh @ kbh.T)
    if bias is not None:
        s = s + bias
    return np.where(keep, s, -np.inf)


def _softmax_rows(s):
    """Row softmax of a score block with ``-inf`` for hidden keys.

    Returns ``(P, lse)``; a row whose keys are all hidden gets ``P = 0`` and
    ``lse = -inf``.
    """
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    ref = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - ref[:, None])
    den = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(den > 0, ref + np.log(den), -np.inf)
        P = np.where(den[:, None] > 0, e / den[:, None], 0.0)
    return P, lse


def attention(q, k, v, scale, causal=False, key_padding_mask=None,
              alibi_slopes=None, rows=None):
    """Exact attention by its definition, one full score matrix per (b, h).

    q: ``[B, S_q, H_q, D]``; k, v: ``[B, S_k, H_kv, D]``; key_padding_mask:
    ``[B, S_k]`` (nonzero keeps) or None; alibi_slopes: ``[H_q]`` or None;
    rows: optional query-row indices to evaluate (the causal rule and the bias
    still use their absolute positions).

    Returns ``out [B, R, H_q, D]`` and ``lse [B, H_q, R]`` in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S_q, H_q, D = q.shape
    S_k, H_kv = k.shape[1], k.shape[2]
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    rows = np.arange(S_q) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    out = np.zeros((B, R, H_q, D))
    lse = np.full((B, H_q, R), -np.inf)
    for b in range(B):
        mrow = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        keep = visible(S_q, S_k, causal, mrow, rows)
        for h in range(H_q):
            hk = h // G
            bias = None
            if alibi_slopes is not None:
                bias = alibi_bias(np.asarray(alibi_slopes, np.float64)[h], S_q, S_k, rows)
            s = _scores(q[b, rows, h, :], k[b, :, hk, :], scale, keep, bias)
            P, lse[b, h] = _softmax_rows(s)
            out[b, :, h, :] = P @ v[b, :, hk, :]
    return out, lse


def attention_ext(q, k, v, scale, causal=False, key_padding_mask=None, alibi_slopes=None,
                  attn_bias=None, dropout_p=0.0, seed=0, offset=0, rows=None):
    """``attention`` with an additive float mask and dropout.

    The forward of the "StreamAttention" page with its additive masks and
    deterministic Philox dropout ("Recent Updates"; ``attention_mask`` and
    ``dropout_p`` of ``forward`` in "API Reference"):

    * ``attn_bias`` (broadcastable to ``[B, H_q, S_q, S_k]``) is added to the
      scaled scores next to the ALiBi bias; ``-inf`` hides a key;
    * the softmax, and so ``lse``, is that of the scores before dropout;
    * with ``dropout_p > 0`` each probability is kept or zeroed by the Philox
      rule of ``oracle.philox.keep_mask`` and the kept ones are divided by
      ``1 - dropout_p``, so ``out_i = sum_j P[i, j] keep[i, j] v_j / (1 - p)``.

    Returns ``out [B, R, H_q, D]`` and ``lse [B, H_q, R]`` in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S_q, H_q, D = q.shape
    S_k, H_kv = k.shape[1], k.shape[2]
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    rows = np.arange(S_q) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    ab = None if attn_bias is None else np.broadcast_to(_f64(attn_bias), (B, H_q, S_q, S_k))
    p = float(dropout_p)
    philox.drop_threshold(p)  # validates p
    out = np.zeros((B, R, H_q, D))
    lse = np.full((B, H_q, R), -np.inf)
    for b in range(B):
        mrow = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        keep = visible(S_q, S_k, causal, mrow, rows)
        for h in range(H_q):
            hk = h // G
            bias = np.zeros((R, S_k))
            if alibi_slopes is not None:
                bias = bias + alibi_bias(np.asarray(alibi_slopes, np.float64)[h], S_q, S_k, rows)
            if ab is not None:
                bias = bias + ab[b, h][rows]
            s = _scores(q[b, rows, h, :], k[b, :, hk, :], scale, keep, bias)
            P, lse[b, h] = _softmax_rows(s)
            if p > 0.0:
                P = P * philox.keep_mask(b, h, H_q, rows, S_k, p, seed, offset) / (1.0 - p)
            out[b, :, h, :] = P @ v[b, :, hk, :]
    return out, lse


# Block size of the block-sparse selection: the default attention block of
# the "Stem: Rethinking Causal Information Flow in Sparse Attention" page
# (section 6, parameter table, ``block_size``), for query rows and keys alike.
SPARSE_BLOCK = 128


def expand_block_mask(block_mask_bh, S_q, S_k, rows=None, block=SPARSE_BLOCK):
    """``[R, S_k]`` boolean: row i may see key j when the block pair
    ``(i // block, j // block)`` is selected in ``block_mask_bh``
    (``[ceil(S_q / block), ceil(S_k / block)]``, nonzero = selected)."""
    rows = np.arange(S_q) if rows is None else np.asarray(rows)
    bm = np.asarray(block_mask_bh) != 0
    return bm[rows // block][:, np.arange(S_k) // block]


def block_sparse_attention(q, k, v, scale, block_mask, causal=False,
                           key_padding_mask=None, alibi_slopes=None, rows=None,
                           block=SPARSE_BLOCK):
    """Attention restricted to selected (query block, key block) pairs.

    The execution step of the "Stem" page (section 2.3, "Block-Sparse
    Attention"): each block of query rows attends only to the key blocks
    chosen for it.  Its fallback, the "pseudo-sparse" run, expands the block
    selection into an element mask and runs dense attention; that is what this
    function does, so a row sees key j when j passes the causal rule and the
    padding mask of ``attention`` *and* j's block is selected for the row's
    block.  ``block_mask``: ``[B, H_q, ceil(S_q / block), ceil(S_k / block)]``,
    nonzero = selected.  A row left with no visible key gets out = 0 and
    lse = -inf.  Returns ``out [B, R, H_q, D]`` and ``lse [B, H_q, R]``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S_q, H_q, D = q.shape
    S_k, H_kv = k.shape[1], k.shape[2]
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    bm = np.asarray(block_mask)
    nbq, nbk = -(-S_q // block), -(-S_k // block)
    if bm.shape != (B, H_q, nbq, nbk):
        raise ValueError(f"block_mask shape {bm.shape} != {(B, H_q, nbq, nbk)}")
    G = H_q // H_kv
    rows = np.arange(S_q) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    out = np.zeros((B, R, H_q, D))
    lse = np.full((B, H_q, R), -np.inf)
    for b in range(B):
        mrow = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        keep = visible(S_q, S_k, causal, mrow, rows)
        for h in range(H_q):
            hk = h // G
            keep_h = keep & expand_block_mask(bm[b, h], S_q, S_k, rows, block)
            bias = None
            if alibi_slopes is not None:
                bias = alibi_bias(np.asarray(alibi_slopes, np.float64)[h], S_q, S_k, rows)
            s = _scores(q[b, rows, h, :], k[b, :, hk, :], scale, keep_h, bias)
            P, lse[b, h] = _softmax_rows(s)
            out[b, :, h, :] = P @ v[b, :, hk, :]
    return out, lse


def online_attention(q, k, v, scale, causal=False, key_padding_mask=None,
                     alibi_slopes=None, block=64):
    """The streaming recurrence of the pages, in float64.

    For each row it keeps a running maximum, a running numerator vector and a
    running denominator; each key block moves the maximum up, rescales both
    running sums by ``exp(old_max - new_max)`` and adds the block's
    ``exp(score - new_max)`` terms ("StreamAttention" page, section "Kernel
    Design"; "Attention API" page, ``online_softmax_attention``).  The
    reference point is 0 while a row has seen no visible key, so no
    ``exp(-inf - (-inf))`` arises ("flash-attn-volta" page, "Stability").
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S_q, H_q, D = q.shape
    S_k, H_kv = k.shape[1], k.shape[2]
    G = H_q // H_kv
    out = np.zeros((B, S_q, H_q, D))
    lse = np.full((B, H_q, S_q), -np.inf)
    for b in range(B):
        mrow = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        keep_all = visible(S_q, S_k, causal, mrow)
        for h in range(H_q):
            hk = h // G
            bias_all = None
            if alibi_slopes is not None:
                bias_all = alibi_bias(np.asarray(alibi_slopes, np.float64)[h], S_q, S_k)
            run_max = np.full(S_q, -np.inf)
            num = np.zeros((S_q, D))
            den = np.zeros(S_q)
            for n0 in range(0, S_k, block):
                n1 = min(n0 + block, S_k)
                bias = None if bias_all is None else bias_all[:, n0:n1]
                s = _scores(q[b, :, h, :], k[b, n0:n1, hk, :], scale,
                            keep_all[:, n0:n1], bias)
                new_max = np.maximum(run_max, s.max(axis=1))
                ref = np.where(np.isfinite(new_max), new_max, 0.0)
                alpha = np.exp(run_max - ref)
                p = np.exp(s - ref[:, None])
                num = alpha[:, None] * num + p @ v[b, n0:n1, hk, :]
                den = alpha * den + p.sum(axis=1)
                run_max = new_max
            with np.errstate(divide="ignore", invalid="ignore"):
                out[b, :, h, :] = np.where(den[:, None] > 0, num / den[:, None], 0.0)
                lse[b, h] = np.where(den > 0, run_max + np.log(den), -np.inf)
    return out, lse


def merge_states(o_parts, lse_parts):
    """Log-sum-exp weighted combination of partial states.

    ``o_parts [P, ..., D]`` are outputs each normalised over its own key subset
    and ``lse_parts [P, ...]`` their log-sum-exps.  The merged
    ``lse = log(sum_p exp(lse_p))`` and ``out = sum_p exp(lse_p - lse) * o_p``;
    parts with ``lse_p = -inf`` contribute nothing, and if all are empty the
    result is ``out = 0``, ``lse = -inf``.
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    M = lse_parts.max(axis=0)
    ref = np.where(np.isfinite(M), M, 0.0)
    w = np.exp(lse_parts - ref[None])
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(tot > 0, ref + np.log(tot), -np.inf)
        wn = np.where(tot[None] > 0, w / tot[None], 0.0)
    out = (wn[..., None] * o_parts).sum(axis=0)
    return out, lse


def attention_bwd(q, k, v, dout, scale, causal=False, key_padding_mask=None,
                  alibi_slopes=None):
    """Gradients of the attention output by its definition, in float64.

    The single-sweep backward of the "StreamAttention: Fused Online Softmax
    Attention" page ("Recent Updates", "Backward": recompute the score tiles
    from the saved lse and stream dQ, dK and dV) and of the "flash-attn-volta"
    page ("Backward correctness") computes these same quantities.  With
    ``P = softmax(s)`` over the visible keys of each row and ``out = P v``:

    * ``dv_j  = sum_i P[i, j] dout_i``
    * ``dP[i, j] = <dout_i, v_j>``
    * ``Di    = sum_j P[i, j] dP[i, j]  ( = <dout_i, out_i> )``
    * ``dS[i, j] = P[i, j] (dP[i, j] - Di)``
    * ``dq_i  = scale * sum_j dS[i, j] k_j``,  ``dk_j = scale * sum_i dS[i, j] q_i``

    Hidden keys have ``P = 0`` and get no gradient from that row; the bias
    and the mask carry no gradient.  A key/value head receives the sum over
    the query heads that read it.  Returns ``dq [B, S_q, H_q, D]``,
    ``dk, dv [B, S_k, H_kv, D]``.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, S_q, H_q, D = q.shape
    S_k, H_kv = k.shape[1], k.shape[2]
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        mrow = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        keep = visible(S_q, S_k, causal, mrow)
        for h in range(H_q):
            hk = h // G
            bias = None
            if alibi_slopes is not None:
                bias = alibi_bias(np.asarray(alibi_slopes, np.float64)[h], S_q, S_k)
            P, _ = _softmax_rows(_scores(q[b, :, h, :], k[b, :, hk, :], scale, keep, bias))
            dqh, dkh, dvh = _bwd_head(P, dout[b, :, h, :], q[b, :, h, :], k[b, :, hk, :],
                                      v[b, :, hk, :], float(scale))
            dq[b, :, h, :] = dqh
            dk[b, :, hk, :] += dkh
            dv[b, :, hk, :] += dvh
    return dq, dk, dv


def _bwd_head(P, do, qh, kh, vh, scale):
    """Gradients of one (batch, query head) from its probabilities ``P``."""
    dv = P.T @ do
    dP = do @ vh.T
    Di = (P * dP).sum(axis=1)
    dS = P * (dP - Di[:, None])
    return scale * (dS @ kh), scale * (dS.T @ qh), dv
