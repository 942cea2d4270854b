#!/usr/bin/env python3
"""Benchmark of the streaming-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over resident synthetic inputs:

* the prefill forward on the 2 x 8192 x 32 x 128 bf16 causal workload with
  ALiBi and a random padding tail (every prefill step: Q tile, K/V streaming,
  scores, bias and masks, online softmax, output and lse), then
* the GQA decode (split-KV + log-sum-exp merge) of 4 sequences over a 32768
  key cache, 14 query heads on 2 KV heads, D = 64, fp16.  Decode steps rotate
  over 8 distinct caches (512 MiB) so the 256 MB last-level cache cannot serve
  one step from the previous one.

``value`` is the step's algorithmic FLOPs (4 * D * H_q * visible query-key
pairs, summed over the parts) divided by the measured time per step, in
TFLOP/s; HIP events on the launch stream bracket the K timed steps, with no
event between the parts of a step.  Each part is then timed on its own: K
calls back to back between two events, after the warm-up count of calls
(and, for a part shorter on the device than its host launch, the decode, a
lead of matrix multiplies so that the device never waits for the host).
Ahead of the warm-up and timed steps bench.py queues at least 150 ms of
4096^3 fp16 matrix multiplies, so that the device never waits for the host
and the timed steps run at the clock sustained work holds, not in the ramp
that follows an idle gap.
The ``roofline`` object is for the dominant kernel (the prefill kernel)
against the 2.5 PFLOP/s dense bf16 matrix peak, and ``decode`` carries the
decode part's key/value read bandwidth against 8 TB/s.  ``cpu_baseline`` times the
float64 CPU oracle on a bounded sample of the same workloads on this host.

The ``*_sparse`` workload times the block-sparse forward
(``sa_attn_fwd_block_sparse``) on the same inputs with a seeded selection of
128 x 128 blocks shaped like the Stem page's (4 sink blocks, a 4-block
window, 20 % of the rest); its FLOPs count only the visible pairs of the
selected blocks.

The ``*_ext`` workload times the extended forward (``sa_attn_fwd_ext``) with
a seeded [B, 1, S_q, S_k] float32 bias and dropout 0.1; its FLOPs are the
forward's (a bias entry of -inf still costs its score).

The ``*_bwd`` workloads time the backward instead (``sa_attn_bwd``: the
per-row pre-pass, the dq kernel and the dk/dv kernel) on the same inputs,
with ``out`` and ``lse`` from one forward call made before timing.  Their
FLOPs are the five products per visible query-key pair (S recomputed, dP, dV,
dK, dQ: 10 * D per pair, 2.5 times the forward's count), and their
``roofline`` is the whole call against the matrix peak.

Prints one JSON line on stdout.  Only one GPU is supported: --gpus above 1
exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "prefill fwd TFLOP/s + decode KV HBM GB/s, each as % of MI355X roofline"
MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix peak (published)
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E bandwidth (published)
# Decode steps rotate over copies of the cache totalling at least this many
# bytes (three times the 256 MB last-level cache), and at least 8 copies.
DECODE_ROTATION_BYTES = 768 << 20
# Least device time of the matrix-multiply lead queued ahead of the timed steps.
PREHEAT_MS = 150.0
PROFILES = ROOT / "profiles"
# Sources each kernel is built from: a traffic figure measured on other sources is stale.
# Each mode of an entry point has its own kernel instances and so its own
# counter summary (``profiles/<tag>_<workload>_traffic.txt``).
KERNEL_SOURCES = {
    "fwd_kernel": ["common.hpp", "host_logic.hpp", "launch.hpp", "prefill.hpp", "sa_attn.hip"],
    "fwd_kernel_sparse": ["common.hpp", "host_logic.hpp", "launch.hpp", "prefill.hpp", "sa_attn_sparse.hip"],
    "fwd_kernel_ext": ["common.hpp", "host_logic.hpp", "launch.hpp", "prefill.hpp", "sa_attn_ext.hip"],
    "decode_kernel": ["common.hpp", "host_logic.hpp", "launch.hpp", "decode.hpp", "sa_attn.hip"],
    "decode_kernel_fused": ["common.hpp", "host_logic.hpp", "launch.hpp", "decode.hpp", "sa_attn.hip"],
    "bwd_kernels": ["common.hpp", "host_logic.hpp", "launch.hpp", "backward.hpp", "sa_attn_bwd.hip"],
}

STEPS = {
    "c5+c4": ["c5_alibi_8192", "c4_decode_32k"],
    "c3_causal_4096": ["c3_causal_4096"],
    "c3_noncausal_4096": ["c3_noncausal_4096"],
    "c5_alibi_8192": ["c5_alibi_8192"],
    "c4_decode_32k": ["c4_decode_32k"],
    "c4_decode_32k_fused": ["c4_decode_32k:fused"],
    "decode_32k_b1": ["decode_32k_b1"],
    "decode_32k_b1_fused": ["decode_32k_b1:fused"],
    "decode_32k_b2": ["decode_32k_b2"],
    "decode_32k_b2_fused": ["decode_32k_b2:fused"],
    "c2_causal_pad16": ["c2_causal_pad16"],
    "c1_fwd_256": ["c1_fwd_256"],
    "c5_alibi_8192_sparse": ["c5_alibi_8192:sparse"],
    "c3_causal_4096_ext": ["c3_causal_4096:ext"],
    "c3_causal_4096_bwd": ["c3_causal_4096:bwd"],
    "c5_alibi_8192_bwd": ["c5_alibi_8192:bwd"],
}


def visible_pairs(w, tails):
    """Query-key pairs the method must visit (causal rule and padding tails)."""
    import numpy as np
    total = 0
    i = np.arange(w.S_q, dtype=np.int64)
    for b in range(w.B):
        t = tails[b] if tails else 0
        last_valid = w.S_k - t - 1
        last = i + (w.S_k - w.S_q) if w.causal else np.full_like(i, w.S_k - 1)
        last = np.minimum(last, last_valid)
        total += int(np.clip(last + 1, 0, None).sum())
    return total


def algorithmic_flops(w, tails, bwd=False):
    """4 * D FLOPs per visible pair forward (two products), 10 * D backward (five)."""
    return (10 if bwd else 4) * w.D * w.H_q * visible_pairs(w, tails)


def sparse_row_block_keys(w, tails, rows=None, block=128):
    """[B, R, nbk]: keys of key block y that row i may see under the causal
    rule and the padding tail (before the block selection)."""
    import numpy as np
    rows = np.arange(w.S_q) if rows is None else np.asarray(rows)
    nbk = -(-w.S_k // block)
    y0 = np.arange(nbk) * block
    out = np.zeros((w.B, len(rows), nbk), dtype=np.int64)
    for b in range(w.B):
        t = tails[b] if tails else 0
        last = np.full(len(rows), w.S_k - t - 1)
        if w.causal:
            last = np.minimum(last, rows + (w.S_k - w.S_q))
        out[b] = np.clip(last[:, None] + 1 - y0[None, :], 0, block)
    return out


def sparse_flops(w, tails, bm, rows=None, block=128):
    """4 * D per visible pair of the selected blocks (bm: [B, H_q, nbq, nbk])."""
    import numpy as np
    rows = np.arange(w.S_q) if rows is None else np.asarray(rows)
    cnt = sparse_row_block_keys(w, tails, rows, block)          # [B, R, nbk]
    sel = np.asarray(bm)[:, :, rows // block, :].astype(np.int64)  # [B, H, R, nbk]
    return 4 * w.D * int((sel * cnt[:, None]).sum())


def kv_bytes(w):
    return 2 * w.B * w.S_k * w.H_kv * w.D * 2


def source_sha(kernel):
    h = hashlib.sha256()
    for n in KERNEL_SOURCES[kernel]:
        h.update((ROOT / "online_softmax_amd" / "csrc" / n).read_bytes())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary of this kernel
    tag (entry-point mode) and workload, if it exists and its sources are
    unchanged; otherwise None."""
    p = PROFILES / f"{kernel}_{workload}_traffic.txt"
    if not p.exists():
        return None
    kv = {}
    for line in p.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha") != source_sha(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Part:
    def __init__(self, name, dev):
        import torch
        import online_softmax_amd as sa
        from workloads import WORKLOADS, make_bias, make_block_mask, make_dout, make_inputs
        name, _, mode = name.partition(":")
        self.bwd = mode == "bwd"
        self.sparse = mode == "sparse"
        self.ext = mode == "ext"
        self.fused = mode == "fused"
        self.w = w = WORKLOADS[name]
        self.sa = sa
        inp = make_inputs(w)
        self.tails = inp.tails
        d = lambda t: None if t is None else t.to(dev)
        self.q, self.mask, self.slopes = d(inp.q), d(inp.mask), d(inp.slopes)
        if w.decode:
            n_rot = max(8, -(-DECODE_ROTATION_BYTES // kv_bytes(w)))
            self.ks = [d(inp.k)] + [d(inp.k).clone() for _ in range(n_rot - 1)]
            self.vs = [d(inp.v)] + [d(inp.v).clone() for _ in range(n_rot - 1)]
            self.ws = (sa.decode_fused_workspace if self.fused else sa.decode_workspace)(
                w.B, w.H_q, w.S_k, w.D, dev)
            self.lse = torch.empty((w.B, w.H_q, 1), dtype=torch.float32, device=dev)
        else:
            self.ks, self.vs = [d(inp.k)], [d(inp.v)]
            self.lse = torch.empty((w.B, w.H_q, w.S_q), dtype=torch.float32, device=dev)
        self.out = torch.empty_like(self.q)
        self.flops = algorithmic_flops(w, self.tails, self.bwd)
        self.calls = 0
        if self.ext:
            self.bias_cpu = make_bias(w, "b1qk")
            self.bias = d(self.bias_cpu)
            self.dropout_p, self.seed = 0.1, 2024
        if self.sparse:
            self.bm_cpu = make_block_mask(w)
            self.bm = d(self.bm_cpu)
            self.flops = sparse_flops(w, self.tails, self.bm_cpu.numpy())
        if self.bwd:
            sa.attn_fwd(self.q, self.ks[0], self.vs[0], causal=w.causal, scale=w.scale,
                        key_padding_mask=self.mask, alibi_slopes=self.slopes, out=self.out,
                        lse=self.lse)
            self.dout = d(make_dout(w))
            self.dq = torch.empty_like(self.q)
            self.dk, self.dv = torch.empty_like(self.ks[0]), torch.empty_like(self.vs[0])
            self.ws = torch.empty(sa.bwd_workspace_size(w.B, w.H_q, w.S_q), dtype=torch.uint8,
                                  device=dev)
        del inp

    def run(self):
        w, i = self.w, self.calls % len(self.ks)
        self.calls += 1
        if self.bwd:
            self.sa.attn_bwd(self.q, self.ks[0], self.vs[0], self.out, self.dout, self.lse,
                             causal=w.causal, scale=w.scale, key_padding_mask=self.mask,
                             alibi_slopes=self.slopes, dq=self.dq, dk=self.dk, dv=self.dv,
                             workspace=self.ws)
        elif self.ext:
            self.sa.attn_fwd_ext(self.q, self.ks[0], self.vs[0], causal=w.causal, scale=w.scale,
                                 key_padding_mask=self.mask, alibi_slopes=self.slopes,
                                 attn_bias=self.bias, dropout_p=self.dropout_p, seed=self.seed,
                                 offset=self.calls, out=self.out, lse=self.lse)
        elif self.sparse:
            self.sa.attn_fwd_block_sparse(self.q, self.ks[0], self.vs[0], self.bm, causal=w.causal,
                                          scale=w.scale, key_padding_mask=self.mask,
                                          alibi_slopes=self.slopes, out=self.out, lse=self.lse)
        elif w.decode and self.fused:
            self.sa.attn_decode_fused(self.q, self.ks[i], self.vs[i], scale=w.scale,
                                      key_padding_mask=self.mask, alibi_slopes=self.slopes,
                                      out=self.out, lse=self.lse, workspace=self.ws)
        elif w.decode:
            self.sa.attn_decode(self.q, self.ks[i], self.vs[i], scale=w.scale,
                                key_padding_mask=self.mask, alibi_slopes=self.slopes,
                                out=self.out, lse=self.lse, workspace=self.ws)
        else:
            self.sa.attn_fwd(self.q, self.ks[i], self.vs[i], causal=w.causal, scale=w.scale,
                             key_padding_mask=self.mask, alibi_slopes=self.slopes,
                             out=self.out, lse=self.lse)


def cpu_baseline(parts, budget_s):
    """Float64 oracle on a bounded row sample of each part, on this host's cores."""
    import numpy as np
    import oracle
    from workloads import make_inputs, to_f64
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    flops = 0
    secs = 0.0
    samples = []
    part_secs = []
    per_part = budget_s / len(parts)
    for p in parts:
        secs_before = secs
        w = p.w
        inp = make_inputs(w)
        q, k, v = to_f64(inp.q), to_f64(inp.k), to_f64(inp.v)
        mask = None if inp.mask is None else inp.mask.numpy()
        sl = None if inp.slopes is None else inp.slopes.numpy()
        causal = w.causal and not w.decode
        if p.bwd:
            f, t, desc = _cpu_bwd_sample(p, inp, q, k, v, mask, sl, per_part)
            flops, secs = flops + f, secs + t
            samples.append(desc)
            part_secs.append(secs - secs_before)
            continue
        # Grow an evenly spaced row sample until the part has used its budget.
        n_rows, used, done_rows = 1, 0.0, 0
        while used < per_part and done_rows < w.S_q:
            n = min(n_rows, w.S_q - done_rows)
            rows = (np.arange(done_rows, done_rows + n) * 7919) % w.S_q
            t0 = time.perf_counter()
            if p.ext:
                oracle.attention_ext(q, k, v, w.scale, causal=causal, key_padding_mask=mask,
                                     alibi_slopes=sl, attn_bias=p.bias_cpu.double().numpy(),
                                     dropout_p=p.dropout_p, seed=p.seed, rows=rows)
                used += time.perf_counter() - t0
                flops += 4 * w.D * w.H_q * sum(int(np.clip(np.minimum(
                    rows + (w.S_k - w.S_q) if causal else np.full(len(rows), w.S_k - 1),
                    w.S_k - 1 - (inp.tails[b] if inp.tails else 0)) + 1, 0, None).sum()) for b in range(w.B))
                done_rows += n
                n_rows *= 2
                continue
            if p.sparse:
                oracle.block_sparse_attention(q, k, v, w.scale, p.bm_cpu.numpy(), causal=causal,
                                              key_padding_mask=mask, alibi_slopes=sl, rows=rows)
                used += time.perf_counter() - t0
                flops += sparse_flops(w, inp.tails, p.bm_cpu.numpy(), rows)
                done_rows += n
                n_rows *= 2
                continue
            oracle.attention(q, k, v, w.scale, causal=causal, key_padding_mask=mask,
                             alibi_slopes=sl, rows=rows)
            used += time.perf_counter() - t0
            for b in range(w.B):
                t = inp.tails[b] if inp.tails else 0
                lastv = w.S_k - t - 1
                last = rows + (w.S_k - w.S_q) if causal else np.full(len(rows), w.S_k - 1)
                flops += 4 * w.D * w.H_q * int(np.clip(np.minimum(last, lastv) + 1, 0, None).sum())
            done_rows += n
            n_rows *= 2
        secs += used
        part_secs.append(secs - secs_before)
        samples.append(f"{w.name}: {done_rows} of {w.S_q} query rows x all batches and heads")
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(samples) + f" ({secs:.1f} s of float64 numpy)",
            "part_seconds": {p.w.name: round(t, 2) for p, t in zip(parts, part_secs)},
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def _cpu_bwd_sample(p, inp, q, k, v, mask, sl, budget_s):
    """Oracle backward over whole (batch row, query head) pairs until the budget is used."""
    import oracle
    from workloads import make_dout, to_f64
    w = p.w
    do = to_f64(make_dout(w))
    flops, used, n = 0, 0.0, 0
    G = w.H_q // w.H_kv
    while used < budget_s and n < w.B * w.H_q:
        b, h = n % w.B, (n // w.B) % w.H_q
        hk = h // G
        t0 = time.perf_counter()
        oracle.attention_bwd(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, hk:hk + 1], v[b:b + 1, :, hk:hk + 1],
                             do[b:b + 1, :, h:h + 1], w.scale, causal=w.causal,
                             key_padding_mask=None if mask is None else mask[b:b + 1],
                             alibi_slopes=None if sl is None else sl[h:h + 1])
        used += time.perf_counter() - t0
        flops += 10 * w.D * visible_pairs(OneRow(w), [inp.tails[b]] if inp.tails else [])
        n += 1
    return flops, used, f"{w.name} backward: {n} of {w.B * w.H_q} (batch row, head) pairs, whole rows"


def cpu_model():
    """The host CPU's model name (as lscpu reports it), from /proc/cpuinfo."""
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_table():
    """Wall time of the float64 oracle per configuration on this host: with the
    BLAS thread count the process has, and with one thread for the small
    configurations 1, 2 and 4.  Inputs are generated before the clock starts.
    Configurations 3 and 5 are timed on whole (batch, head) pairs until 20 s
    have passed and scaled to all of them (the oracle's cost is the same for
    every pair of a configuration)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    from workloads import WORKLOADS, make_inputs, to_f64
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    rows = []
    for name in ["c1_fwd_256", "c2_causal_pad16", "c3_causal_4096", "c3_noncausal_4096",
                 "c4_decode_32k", "c5_alibi_8192"]:
        w = WORKLOADS[name]
        inp = make_inputs(w)
        q, k, v = to_f64(inp.q), to_f64(inp.k), to_f64(inp.v)
        mask = None if inp.mask is None else inp.mask.numpy()
        sl = None if inp.slopes is None else inp.slopes.numpy()
        causal = w.causal and not w.decode
        small = name in ("c1_fwd_256", "c2_causal_pad16", "c4_decode_32k")

        def whole():
            t0 = time.perf_counter()
            oracle.attention(q, k, v, w.scale, causal=causal, key_padding_mask=mask, alibi_slopes=sl)
            return time.perf_counter() - t0

        def by_pairs(budget=20.0):
            G = w.H_q // w.H_kv
            used, n = 0.0, 0
            while used < budget and n < w.B * w.H_q:
                b, h = n % w.B, (n // w.B) % w.H_q
                t0 = time.perf_counter()
                oracle.attention(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h // G:h // G + 1],
                                 v[b:b + 1, :, h // G:h // G + 1], w.scale, causal=causal,
                                 key_padding_mask=None if mask is None else mask[b:b + 1],
                                 alibi_slopes=None if sl is None else sl[h:h + 1])
                used += time.perf_counter() - t0
                n += 1
            return used * (w.B * w.H_q) / n, n

        if small:
            whole()  # first call: BLAS thread start-up, outside the clock
            t_all = whole()
            with threadpool_limits(1):
                t_one = whole()
            rows.append({"config": name, "all_threads_s": round(t_all, 3), "one_thread_s": round(t_one, 3),
                         "timed": "whole"})
        else:
            t_all, n = by_pairs()
            rows.append({"config": name, "all_threads_s": round(t_all, 2), "one_thread_s": None,
                         "timed": f"{n} of {w.B * w.H_q} (batch, head) pairs, scaled"})
    return {"blas_threads": threads, "host_cpus": os.cpu_count(), "cpu_model": cpu_model(), "rows": rows}


class OneRow:
    """One batch row of a workload (for counting its visible pairs)."""
    def __init__(self, w):
        self.B, self.S_q, self.S_k, self.causal = 1, w.S_q, w.S_k, w.causal


def copy_calibration(args, dev):
    """A plain copy of known size: reads and writes exactly copy_mib MiB each."""
    import torch
    n = args.copy_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes": n, "ms_per_copy": round(dt * 1e3, 4),
                      "read_plus_write_GBs": round(2 * n / dt / 1e9, 1)}), flush=True)


def gemm_calibration(args, dev):
    """A plain bfloat16 matrix product (torch.matmul, n x n x n) for a
    reference of what the matrix cores sustain on this GPU outside attention."""
    import torch
    n = args.gemm
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(args.warmup):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    dt = e0.elapsed_time(e1) / 1e3 / args.steps
    flops = 2.0 * n ** 3
    print(json.dumps({"gemm_n": n, "dtype": "bf16", "ms_per_gemm": round(dt * 1e3, 4),
                      "TFLOPs": round(flops / dt / 1e12, 1),
                      "frac_of_2500": round(flops / dt / 1e12 / MFMA_PEAK_TFLOPS, 4)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c5+c4", choices=sorted(STEPS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--print-source-sha", action="store_true",
                    help="print the source hash of each kernel (recorded with counter summaries) and exit")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--cpu-table", action="store_true",
                    help="instead of the hot path, print the float64 oracle's wall time per configuration "
                         "on this host (all BLAS threads, and one thread for configurations 1, 2 and 4)")
    ap.add_argument("--gemm", type=int, default=0,
                    help="instead of the hot path, time a plain n x n x n bfloat16 torch.matmul")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of the hot path, time a plain device-to-device copy of this many "
                         "MiB (the reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.print_source_sha:
        print(json.dumps({k: source_sha(k) for k in KERNEL_SOURCES}))
        return
    if args.cpu_table:
        print(json.dumps(cpu_table()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "no GPU visible"
    dev = torch.device("cuda:0")
    if args.copy_mib:
        copy_calibration(args, dev)
        return
    if args.gemm:
        gemm_calibration(args, dev)
        return
    parts = [Part(n, dev) for n in STEPS[args.workload]]
    stream = torch.cuda.current_stream(dev)

    # Warm-up: the first steps one at a time (first use of every kernel, and
    # the host's time per step), the rest queued directly ahead of the timed
    # steps, after the lead below.
    n_sync = min(args.warmup, 3)
    host_s = []
    for _ in range(n_sync):
        t0 = time.perf_counter()
        for p in parts:
            p.run()
        host_s.append(time.perf_counter() - t0)
        torch.cuda.synchronize()

    # The device must not wait for the host between steps (a short decode step
    # takes less device time than the Python call that launches it): queue a
    # matrix-multiply lead of known length first, long enough for the host to
    # enqueue the remaining warm-up steps and every timed step before the
    # device reaches them.
    a = torch.randn(4096, 4096, device=dev, dtype=torch.float16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.mm(a, a)
    e0.record(stream)
    torch.mm(a, a)
    e1.record(stream)
    torch.cuda.synchronize()
    mm_ms = max(e0.elapsed_time(e1), 1e-3)
    host_step_s = sorted(host_s)[len(host_s) // 2] if host_s else 1e-3

    def lead(n_calls, host_s_per_call, min_ms=0.0):
        lead_ms = max(1.5 * n_calls * 1e3 * host_s_per_call + 1.0, min_ms)
        n = min(int(math.ceil(lead_ms / mm_ms)), 20000)
        for _ in range(n):
            torch.mm(a, a)
        return n

    # Timed steps: events only before the first and after the last, so that
    # no event marker sits between the parts of a step.  The lead ahead of
    # them is at least PREHEAT_MS of matrix multiplies: after an idle gap the
    # c5 prefill took 1.2-1.4 ms on its first launches and settled at
    # 1.09 ms only after about 25 (the GPU's clock under sustained load),
    # while right after 600 matrix multiplies it settled within 5; so the
    # timed steps run in the state that sustained work keeps the GPU in,
    # whatever the warm-up count.
    t0 = time.perf_counter()
    n_lead = lead(args.warmup - n_sync + args.steps, host_step_s, PREHEAT_MS)
    for _ in range(args.warmup - n_sync):
        for p in parts:
            p.run()
    e0.record(stream)
    for s in range(args.steps):
        for p in parts:
            p.run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = max(e0.elapsed_time(e1) / args.steps, 0.0)

    # Each part's own time per call, right after the timed steps: the same
    # number of calls back to back between two events, after the warm-up
    # count of calls.  A part that takes less device time per call than the
    # host needs to launch it (the decode) gets a lead first; the prefill,
    # which the lead's matrix multiplies would slow for its next launches,
    # does not need one.
    part_ms = []
    for p in parts:
        torch.cuda.synchronize()
        t_host = time.perf_counter()
        e0.record(stream)
        for _ in range(3):
            p.run()
        e1.record(stream)
        host_call_s = (time.perf_counter() - t_host) / 3
        torch.cuda.synchronize()
        if e0.elapsed_time(e1) / 3 < 2e3 * host_call_s:
            lead(args.warmup + args.steps, host_call_s)
        for _ in range(args.warmup):
            p.run()
        e0.record(stream)
        for _ in range(args.steps):
            p.run()
        e1.record(stream)
        torch.cuda.synchronize()
        part_ms.append(e0.elapsed_time(e1) / args.steps)

    total_flops = sum(p.flops for p in parts)
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    result = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": parts[0].w.dtype if parts[0].w.dtype != "fp16" else "fp16",
        "data": "synthetic (seeded N(0,1) q/k/v)",
        "config": {"workload": args.workload,
                   "parts": [f"{p.w.name}{' backward' if p.bwd else ''}"
                             f"{' + [B,1,S_q,S_k] float bias + dropout %.1f' % p.dropout_p if p.ext else ''}"
                             f"{' block-sparse (%.1f %% of blocks selected)' % (100 * p.bm_cpu.float().mean().item()) if p.sparse else ''}: B={p.w.B} S_q={p.w.S_q} S_k={p.w.S_k} H_q={p.w.H_q} "
                             f"H_kv={p.w.H_kv} D={p.w.D} {p.w.dtype} causal={p.w.causal} "
                             f"mask={'tails ' + str(p.tails) if p.tails else 'none'} "
                             f"alibi={p.w.alibi}" for p in parts],
                   "wall_s_lead_warmup_timed": round(wall, 4),
                   "device_lead_ms": round(n_lead * mm_ms, 3)},
    }
    prefill = [(p, t) for p, t in zip(parts, part_ms) if not p.w.decode and not p.bwd]
    decode = [(p, t) for p, t in zip(parts, part_ms) if p.w.decode]
    backward = [(p, t) for p, t in zip(parts, part_ms) if p.bwd]
    if backward:
        p, t = backward[0]
        ach = p.flops / (t * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS, 4),
                              "traffic": read_traffic("bwd_kernels", p.w.name),
                              "kernel": "bwd_dq_kernel + bwd_dkdv_kernel (one call)",
                              "workload": p.w.name + " backward", "avg_call_ms": round(t, 4),
                              "flops_per_call": p.flops}
    if prefill:
        p, t = max(prefill, key=lambda x: x[1])
        ach = p.flops / (t * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS, 4),
                              "traffic": read_traffic("fwd_kernel" + ("_sparse" if p.sparse else "")
                                                      + ("_ext" if p.ext else ""), p.w.name),
                              "kernel": "fwd_kernel" + (" (block-sparse)" if p.sparse else "")
                                        + (" (bias + dropout)" if p.ext else ""),
                              "workload": p.w.name + (" block-sparse" if p.sparse else "")
                                          + (" bias + dropout" if p.ext else ""),
                              "avg_launch_ms": round(t, 4), "flops_per_launch": p.flops,
                              "dense_count_tflops": round(4 * p.w.B * p.w.H_q * p.w.S_q * p.w.S_k * p.w.D
                                                          / (t * 1e-3) / 1e12, 2)}
    if decode:
        p, t = decode[0]
        gbs = kv_bytes(p.w) / (t * 1e-3) / 1e9
        dec = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": read_traffic("decode_kernel" + ("_fused" if p.fused else ""), p.w.name),
               "kernels": "decode_kernel (single-kernel mode)" if p.fused else "decode_kernel + decode_merge_kernel",
               "workload": p.w.name + (" single-kernel" if p.fused else ""),
               "avg_call_us": round(t * 1e3, 2), "kv_bytes_per_call": kv_bytes(p.w)}
        if prefill:
            result["decode"] = dec
        else:
            result["roofline"] = dec
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(parts, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
