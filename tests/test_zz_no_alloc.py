"""GPU test of the allocation-free decode (sa_attn_decode_noalloc), called
through the C ABI: its outputs equal those of sa_attn_decode (same kernels,
same split count; the library's scratch in place of a workspace) bit for bit,
and both match the oracle, on two calls in a row, the second smaller than the
first (the scratch keeps the first call's partial results, which the second
must not read)."""
import ctypes

import numpy as np
import pytest
import torch

import online_softmax_amd as sa
from parity import assert_lse_close, assert_out_close, oracle_for, p_rounding, to_dev
from workloads import WORKLOADS, Workload, make_inputs, to_f64

pytestmark = pytest.mark.gpu


def _noalloc(inp, out, lse):
    w = inp.w
    q, k, v, m, s = to_dev(inp)
    L = sa.lib()
    st = L.sa_attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                  w.B, w.S_k, w.H_q, w.H_kv, w.D, w.scale,
                                  None if m is None else m.data_ptr(), None if s is None else s.data_ptr(),
                                  0 if w.dtype == "fp16" else 1, torch.cuda.current_stream().cuda_stream)
    assert st == sa.SA_OK, sa.last_error()
    torch.cuda.synchronize()


def test_noalloc_matches_decode_twice():
    big = WORKLOADS["c4_decode_32k"]
    small = Workload("noalloc_small", 2, 1, 3000, 8, 2, 128, "bf16", alibi=True, random_tail=500, seed=181)
    for w in (big, small):
        inp = make_inputs(w)
        print(f"[noalloc] {w.name} B={w.B} S_k={w.S_k} H={w.H_q}/{w.H_kv} D={w.D} {w.dtype}", flush=True)
        q, k, v, m, s = to_dev(inp)
        want_o, want_l = sa.attn_decode(q, k, v, scale=w.scale, key_padding_mask=m, alibi_slopes=s)
        out = torch.full_like(want_o, float("nan"))
        lse = torch.full_like(want_l, float("nan"))
        _noalloc(inp, out, lse)
        assert torch.equal(out, want_o) and torch.equal(lse, want_l)
        ref_o, ref_l = oracle_for(inp, causal=False)
        dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
        assert_out_close(to_f64(out.cpu()), ref_o, dt, w.name,
                         p_rounding(oracle_for(inp, causal=False, abs_v=True)[0], dt))
        assert_lse_close(lse.cpu().double().numpy(), ref_l, w.name)


def test_noalloc_rejects_beyond_scratch():
    """A decode whose partial results exceed the 16 MiB scratch is refused
    with a message (no launch)."""
    B, S_k, H_q, H_kv, D = 64, 128, 512, 512, 128   # 64 * 512 * 1 * 129 * 4 B = 16.9 MB
    q = torch.zeros((B, 1, H_q, D), dtype=torch.float16, device="cuda")
    kv = torch.zeros((B, S_k, H_kv, D), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q)
    L = sa.lib()
    st = L.sa_attn_decode_noalloc(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), out.data_ptr(), None,
                                  B, S_k, H_q, H_kv, D, 0.1, None, None, 0, None)
    assert st == sa.SA_ERR_UNSUPPORTED and "scratch" in sa.last_error()
