"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random tensors and builds masks and slope vectors; it holds
none of the attention arithmetic.  Both the HIP path and the CPU oracle are fed
from here, and neither imports the other.

Recipe (the same for every named workload): ``g = torch.Generator().manual_seed(seed)``,
then ``q``, ``k``, ``v`` drawn in that order with ``torch.randn`` in float32 at
their ``[B, S, H, D]`` shapes and cast to fp16 or bf16; a random padding tail,
when the workload has one, is drawn next with ``torch.randint``.  ALiBi slopes
follow the geometric sequence ``2^(-8 (h + 1) / H)`` over zero-based heads,
rounded to float32; the softmax scale is ``float32(1 / sqrt(D))``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S_q: int
    S_k: int
    H_q: int
    H_kv: int
    D: int
    dtype: str = "fp16"
    causal: bool = False
    pad_tail: int = 0          # fixed number of masked keys at the end of every batch row
    random_tail: int = 0       # masked tail drawn per batch row from randint(0, random_tail + 1)
    alibi: bool = False
    seed: int = 0
    decode: bool = False       # S_q == 1 through the split-KV decode entry point
    note: str = ""

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def has_mask(self) -> bool:
        return self.pad_tail > 0 or self.random_tail > 0


# The five named workloads.  Shapes follow the pages' own workloads: the
# accuracy CLI shape and the quick-start mask of the "StreamAttention" page,
# the 4096-token rows of the "flash-attn-volta" forward benchmark, a Qwen2.5-0.5B
# style 14:2 GQA decode over a 32K cache, and the quick-start 32-head,
# 128-wide configuration at batch 2.
WORKLOADS = {
    "c1_fwd_256": Workload("c1_fwd_256", 1, 256, 256, 4, 4, 64, "fp16", seed=1,
                           note="non-causal, no mask"),
    "c2_causal_pad16": Workload("c2_causal_pad16", 2, 1024, 1024, 8, 8, 64, "fp16",
                                causal=True, pad_tail=16, seed=2,
                                note="causal, last 16 keys of each batch row masked"),
    "c3_causal_4096": Workload("c3_causal_4096", 1, 4096, 4096, 16, 16, 128, "fp16",
                               causal=True, seed=3, note="causal"),
    "c3_noncausal_4096": Workload("c3_noncausal_4096", 1, 4096, 4096, 16, 16, 128, "fp16",
                                  causal=False, seed=3, note="non-causal variant of c3"),
    "c4_decode_32k": Workload("c4_decode_32k", 4, 1, 32768, 14, 2, 64, "fp16",
                              seed=4, decode=True,
                              note="GQA 7:1 decode, all 32768 keys valid"),
    # The same decode at the small batches the single-kernel decode is for.
    "decode_32k_b1": Workload("decode_32k_b1", 1, 1, 32768, 14, 2, 64, "fp16", seed=4, decode=True,
                              note="c4_decode_32k at batch 1"),
    "decode_32k_b2": Workload("decode_32k_b2", 2, 1, 32768, 14, 2, 64, "fp16", seed=4, decode=True,
                              note="c4_decode_32k at batch 2"),
    "c5_alibi_8192": Workload("c5_alibi_8192", 2, 8192, 8192, 32, 32, 128, "bf16",
                              causal=True, random_tail=512, alibi=True, seed=5,
                              note="causal + ALiBi + random padding tail"),
}


def alibi_slopes(H: int) -> torch.Tensor:
    """float32 ``[H]`` slopes ``2^(-8 (h + 1) / H)``, h = 0 .. H-1."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)],
                        dtype=torch.float32)


@dataclass
class Inputs:
    w: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    mask: Optional[torch.Tensor]      # uint8 [B, S_k], 1 = keep, or None
    slopes: Optional[torch.Tensor]    # float32 [H_q] or None
    tails: list = field(default_factory=list)


def make_inputs(w: Workload, seed: Optional[int] = None, scale_qk: float = 1.0) -> Inputs:
    """CPU tensors for workload ``w`` (seed defaults to the workload's own).

    ``scale_qk`` multiplies the float32 draws of q and k before the cast,
    which the overflow cases use to push ``q . k`` past the fp16 range.
    """
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    dt = DTYPES[w.dtype]
    q = torch.randn((w.B, w.S_q, w.H_q, w.D), generator=g)
    k = torch.randn((w.B, w.S_k, w.H_kv, w.D), generator=g)
    v = torch.randn((w.B, w.S_k, w.H_kv, w.D), generator=g)
    if scale_qk != 1.0:
        q, k = q * scale_qk, k * scale_qk
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    mask = None
    tails = []
    if w.has_mask:
        mask = torch.ones((w.B, w.S_k), dtype=torch.uint8)
        if w.random_tail:
            tails = torch.randint(0, w.random_tail + 1, (w.B,), generator=g).tolist()
        else:
            tails = [w.pad_tail] * w.B
        for b, t in enumerate(tails):
            if t:
                mask[b, w.S_k - t:] = 0
    slopes = alibi_slopes(w.H_q) if w.alibi else None
    return Inputs(w, q, k, v, mask, slopes, tails)


def make_dout(w: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """Seeded upstream gradient of the output (``[B, S_q, H_q, D]``, N(0, 1)
    drawn in float32 and cast), for the backward; seed defaults to the
    workload's seed + 1000."""
    g = torch.Generator().manual_seed(w.seed + 1000 if seed is None else seed)
    return torch.randn((w.B, w.S_q, w.H_q, w.D), generator=g).to(DTYPES[w.dtype])


def make_block_mask(w: Workload, keep: float = 0.2, sinks: int = 4, window: int = 4,
                    seed: Optional[int] = None, block: int = 128) -> torch.Tensor:
    """Seeded block selection for the block-sparse forward, shaped like the
    selections of the "Stem" page: per (batch, query head, query block x),
    the first ``sinks`` key blocks and the ``window`` key blocks ending at the
    query block's own diagonal (its section 6 defaults ``initial_blocks`` = 4
    and ``window_size`` = 4) are always selected, and every other key block
    independently with probability ``keep`` (standing in for the top-k of
    its scores).  The diagonal of block x is the key block holding key
    ``x * block + block - 1 + S_k - S_q`` (bottom-right alignment).
    Returns uint8 ``[B, H_q, ceil(S_q / block), ceil(S_k / block)]``.
    """
    g = torch.Generator().manual_seed(w.seed + 2000 if seed is None else seed)
    nbq, nbk = -(-w.S_q // block), -(-w.S_k // block)
    bm = (torch.rand((w.B, w.H_q, nbq, nbk), generator=g) < keep).to(torch.uint8)
    bm[:, :, :, :min(sinks, nbk)] = 1
    for x in range(nbq):
        last = min(x * block + block - 1 + w.S_k - w.S_q, w.S_k - 1)
        if last < 0:
            continue
        d = last // block
        bm[:, :, x, max(0, d - window + 1):d + 1] = 1
    return bm


def make_bias(w: Workload, kind: str = "b1qk", ninf: float = 0.02, seed: Optional[int] = None) -> torch.Tensor:
    """Seeded additive float32 mask: N(0, 1) entries with a fraction ``ninf``
    set to -inf (hidden keys), at one of the broadcast shapes a caller may
    pass: ``bhqk`` [B, H_q, S_q, S_k], ``b1qk`` [B, 1, S_q, S_k], ``qk``
    [S_q, S_k] or ``b11k`` [B, 1, 1, S_k]."""
    g = torch.Generator().manual_seed(w.seed + 3000 if seed is None else seed)
    shape = {"bhqk": (w.B, w.H_q, w.S_q, w.S_k), "b1qk": (w.B, 1, w.S_q, w.S_k),
             "qk": (w.S_q, w.S_k), "b11k": (w.B, 1, 1, w.S_k)}[kind]
    bias = torch.randn(shape, generator=g)
    if ninf > 0:
        bias[torch.rand(shape, generator=g) < ninf] = float("-inf")
    return bias


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 numpy copy of a CPU tensor (fp16/bf16 values are exact in fp64)."""
    return t.detach().to("cpu", torch.float64).numpy()
