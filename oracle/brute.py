"""Scalar pure-Python attention for tiny inputs (test infrastructure only).

The same definition as ``oracle.attention`` written with nested loops over
Python floats, ``math.exp``, ``math.log`` and ``math.fsum``: no numpy, no
matrix products, no vectorised masking.  It shares no helper with the numpy
oracle, so the two agreeing to 1e-12 pins the numpy version's indexing (head
grouping, transposes, bias sign and offset, visibility) on every shape small
enough to run here (sequence lengths up to about 8).
"""
from __future__ import annotations

import math

from .philox import drop_threshold, philox4x32_10


def attention(q, k, v, scale, causal=False, key_padding_mask=None,
              alibi_slopes=None, block_mask=None, block=128, attn_bias=None,
              dropout_p=0.0, seed=0, offset=0):
    """q: nested ``[B][S_q][H_q][D]``; k, v: ``[B][S_k][H_kv][D]``.

    ``block_mask`` (nested ``[B][H_q][query block][key block]``, truthy =
    selected) restricts row i to keys whose block of ``block`` keys is
    selected for the block of ``block`` rows holding i.  ``attn_bias``
    (nested ``[B][H_q][S_q][S_k]``) is added to the scaled score; with
    ``dropout_p > 0`` each term of the output sum is kept when its 16-bit
    Philox value (one generator call per element) reaches the drop
    threshold, and is then divided by ``1 - dropout_p``.

    Returns ``(out [B][S_q][H_q][D], lse [B][H_q][S_q])`` as Python floats.
    """
    B, S_q, H_q, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    S_k, H_kv = len(k[0]), len(k[0][0])
    G = H_q // H_kv
    out = [[[[0.0] * D for _ in range(H_q)] for _ in range(S_q)] for _ in range(B)]
    lse = [[[float("-inf")] * S_q for _ in range(H_q)] for _ in range(B)]
    for b in range(B):
        for h in range(H_q):
            hk = h // G
            for i in range(S_q):
                pos = i + S_k - S_q
                keys, scores = [], []
                for j in range(S_k):
                    if causal and j > pos:
                        continue
                    if key_padding_mask is not None and not key_padding_mask[b][j]:
                        continue
                    if block_mask is not None and not block_mask[b][h][i // block][j // block]:
                        continue
                    dot = math.fsum(float(q[b][i][h][d]) * float(k[b][j][hk][d])
                                    for d in range(D))
                    sc = float(scale) * dot
                    if alibi_slopes is not None:
                        sc -= float(alibi_slopes[h]) * abs(pos - j)
                    if attn_bias is not None:
                        sc += float(attn_bias[b][h][i][j])
                        if sc == float("-inf"):
                            continue
                    keys.append(j)
                    scores.append(sc)
                if not keys:
                    continue
                top = max(scores)
                total = math.fsum(math.exp(x - top) for x in scores)
                row_lse = top + math.log(total)
                lse[b][h][i] = row_lse
                weight = [math.exp(sc - row_lse) for sc in scores]
                if dropout_p > 0.0:
                    thr = drop_threshold(dropout_p)
                    for n, j in enumerate(keys):
                        window, within = divmod(j, 64)
                        word = philox4x32_10((8 * window + (within % 32) // 4, i, b * H_q + h, offset),
                                             (seed & 0xFFFFFFFF, seed >> 32))[within % 4]
                        value = (word >> 16) if within >= 32 else (word & 0xFFFF)
                        weight[n] = weight[n] / (1.0 - dropout_p) if value >= thr else 0.0
                for d in range(D):
                    out[b][i][h][d] = math.fsum(
                        wt * float(v[b][j][hk][d]) for wt, j in zip(weight, keys))
    return out, lse
