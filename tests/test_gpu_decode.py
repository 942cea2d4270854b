"""GPU parity of the split-KV decode path (sa_attn_decode) against the oracle.

The oracle for one query token is the same definition as for prefill with
S_q = 1 (the bottom-right causal rule hides nothing from the last row).
"""
import numpy as np
import pytest
import torch

import online_softmax_amd as sa
from parity import assert_lse_close, assert_out_close, oracle_for, p_rounding, to_dev
from workloads import WORKLOADS, Workload, make_inputs, to_f64

pytestmark = pytest.mark.gpu


def run_decode(inp):
    q, k, v, m, s = to_dev(inp)
    out, lse = sa.attn_decode(q, k, v, scale=inp.w.scale, key_padding_mask=m, alibi_slopes=s)
    torch.cuda.synchronize()
    return to_f64(out.cpu()), lse.cpu().double().numpy()


def check(inp, what=""):
    w = inp.w
    print(f"[decode] {what or w.name} B={w.B} S_k={w.S_k} H={w.H_q}/{w.H_kv} D={w.D} {w.dtype} "
          f"mask={inp.mask is not None} alibi={inp.slopes is not None}", flush=True)
    out, lse = run_decode(inp)
    ref_o, ref_l = oracle_for(inp, causal=False)
    dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    assert_out_close(out, ref_o, dt, what or w.name,
                     p_rounding(oracle_for(inp, causal=False, abs_v=True)[0], dt))
    assert_lse_close(lse, ref_l, what or w.name)
    return out, lse


CASES = [
    Workload("dec_k1", 2, 1, 1, 4, 4, 64, "fp16", seed=40),
    Workload("dec_k100_g7", 3, 1, 100, 14, 2, 64, "fp16", seed=41),
    Workload("dec_k1000_g8_mask", 2, 1, 1000, 16, 2, 128, "bf16", random_tail=400, seed=42),
    Workload("dec_k5000_alibi", 2, 1, 5000, 8, 8, 64, "fp16", alibi=True, seed=43),
    Workload("dec_k777_all", 2, 1, 777, 28, 4, 128, "bf16", alibi=True, random_tail=300, seed=44),
    Workload("dec_g40_two_groups", 1, 1, 300, 40, 1, 64, "fp16", seed=45),
    Workload("dec_k129_mha", 4, 1, 129, 6, 6, 128, "fp16", seed=46),
    # One head group, 256 splits of 128 keys: the widest merge.
    Workload("dec_k32768_256splits", 1, 1, 32768, 4, 1, 128, "bf16", seed=51),
    # Two full head groups of 16 and 300 keys: rounds past the split's end.
    Workload("dec_g32_d128", 2, 1, 300, 32, 1, 128, "fp16", alibi=True, seed=52),
    # Splits of 2048 keys at D = 64: four rounds of loads per workgroup, the
    # last split's last round partly past its end.
    Workload("dec_long_splits", 8, 1, 8000, 16, 8, 64, "bf16", alibi=True, random_tail=2000, seed=64),
    # Splits of 384 keys at D = 128: two rounds, the second with 4 of its 8
    # sub-tiles inside the split.
    Workload("dec_d128_partial_round", 4, 1, 6000, 8, 4, 128, "fp16", random_tail=1500, seed=65),
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_decode_cases(w):
    check(make_inputs(w))


def test_config4_full():
    check(make_inputs(WORKLOADS["c4_decode_32k"]))


def test_decode_empty_cache():
    q = torch.randn(2, 1, 4, 64, device="cuda").half()
    k = torch.zeros(2, 0, 2, 64, device="cuda").half()
    out, lse = sa.attn_decode(q, k, k.clone())
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()


def test_decode_fully_masked_row():
    w = Workload("dec_masked", 2, 1, 500, 4, 2, 64, "fp16", seed=47)
    inp = make_inputs(w)
    inp.mask = torch.ones((2, 500), dtype=torch.uint8)
    inp.mask[0] = 0
    out, lse = check(inp, "fully masked batch row")
    assert (out[0] == 0).all() and np.isneginf(lse[0]).all()


def test_decode_matches_prefill_last_row():
    """Decode of the last query equals row S-1 of a causal prefill on the same K/V."""
    S = 700
    w = Workload("dec_vs_fwd", 2, S, S, 8, 2, 64, "fp16", causal=True, alibi=True, seed=48)
    inp = make_inputs(w)
    q, k, v, m, s = to_dev(inp)
    out_f, lse_f = sa.attn_fwd(q, k, v, causal=True, scale=w.scale, alibi_slopes=s)
    out_d, lse_d = sa.attn_decode(q[:, S - 1:S].contiguous(), k, v, scale=w.scale, alibi_slopes=s)
    torch.cuda.synchronize()
    a, b = out_f[:, S - 1:S].double().cpu().numpy(), out_d.double().cpu().numpy()
    assert np.abs(a - b).max() <= 2e-3
    assert np.abs(lse_f[:, :, S - 1:S].cpu().numpy() - lse_d.cpu().numpy()).max() <= 1e-4


def test_decode_workspace_errors():
    w = Workload("dec_ws", 1, 1, 300, 4, 4, 64, "fp16", seed=49)
    q, k, v, _, _ = to_dev(make_inputs(w))
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(sa.SaAttnError) as e:
        sa.attn_decode(q, k, v, workspace=small)
    assert e.value.status == sa.SA_ERR_WORKSPACE


def test_decode_workspace_reuse():
    """One workspace serves calls of different sizes in a row."""
    ws = sa.decode_workspace(3, 32, 40000, 128, "cuda")
    for i, w in enumerate([Workload("dec_reuse_a", 3, 1, 5000, 14, 2, 64, "fp16", seed=53),
                           Workload("dec_reuse_b", 1, 1, 40000, 32, 4, 128, "bf16", random_tail=900, seed=54),
                           Workload("dec_reuse_c", 2, 1, 700, 8, 8, 64, "fp16", alibi=True, seed=55),
                           Workload("dec_reuse_a", 3, 1, 5000, 14, 2, 64, "fp16", seed=53)]):
        inp = make_inputs(w)
        q, k, v, m, s = to_dev(inp)
        print(f"[decode reuse] call {i}: {w.name}", flush=True)
        out, lse = sa.attn_decode(q, k, v, scale=w.scale, key_padding_mask=m, alibi_slopes=s,
                                  workspace=ws)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_for(inp, causal=False)
        dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
        assert_out_close(to_f64(out.cpu()), ref_o, dt, w.name,
                         p_rounding(oracle_for(inp, causal=False, abs_v=True)[0], dt))
        assert_lse_close(lse.cpu().double().numpy(), ref_l, w.name)


def test_decode_deterministic():
    inp = make_inputs(Workload("dec_det", 2, 1, 3000, 14, 2, 64, "fp16", random_tail=100, seed=50))
    a, b = run_decode(inp), run_decode(inp)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


# ---------------------------------------------------------------- single kernel

FUSED_CASES = [
    Workload("fu_b1_32k", 1, 1, 32768, 14, 2, 64, "fp16", decode=True, seed=56),
    Workload("fu_b2_32k_mask", 2, 1, 32768, 14, 2, 64, "fp16", decode=True, random_tail=900, seed=57),
    Workload("fu_b3_alibi_d128", 3, 1, 5000, 8, 2, 128, "bf16", decode=True, alibi=True, seed=58),
    Workload("fu_b1_g40", 1, 1, 3000, 40, 1, 64, "fp16", decode=True, seed=59),
    Workload("fu_b2_short_all", 2, 1, 129, 28, 4, 128, "bf16", decode=True, alibi=True, random_tail=60, seed=60),
    Workload("fu_b1_k1", 1, 1, 1, 4, 4, 64, "fp16", decode=True, seed=61),
    # 320 head groups of two splits each
    Workload("fu_b40_groups", 40, 1, 700, 32, 8, 64, "bf16", decode=True, random_tail=300, seed=62),
    # two groups of 16 heads at D = 128 over 63 splits: 512 (head, d chunk) pairs,
    # so the merge takes two sweeps of two chunks, the second one ragged
    Workload("fu_b1_g16_d128_40k", 1, 1, 40000, 32, 2, 128, "fp16", decode=True, seed=63),
    # splits of 2048 and 384 keys (several rounds, the last one partial)
    Workload("fu_long_splits", 8, 1, 8000, 16, 8, 64, "bf16", decode=True, alibi=True, random_tail=2000,
             seed=66),
    Workload("fu_d128_partial_round", 4, 1, 6000, 8, 4, 128, "fp16", decode=True, random_tail=1500, seed=67),
]


def counters_clear(ws):
    """Every arrival counter (the first 64 KiB of the single-kernel decode's
    workspace) is back at zero."""
    return bool((ws[:sa.DECODE_ARRIVE_BYTES] == 0).all().item())


def run_fused(inp, ws=None):
    q, k, v, m, s = to_dev(inp)
    out, lse = sa.attn_decode_fused(q, k, v, scale=inp.w.scale, key_padding_mask=m, alibi_slopes=s,
                                    workspace=ws)
    torch.cuda.synchronize()
    return to_f64(out.cpu()), lse.cpu().double().numpy()


@pytest.mark.parametrize("w", FUSED_CASES, ids=lambda w: w.name)
def test_decode_fused_cases(w):
    inp = make_inputs(w)
    print(f"[decode fused] {w.name} B={w.B} S_k={w.S_k} H={w.H_q}/{w.H_kv} D={w.D} {w.dtype}", flush=True)
    ws = sa.decode_fused_workspace(w.B, w.H_q, w.S_k, w.D, "cuda")
    out, lse = run_fused(inp, ws)
    assert counters_clear(ws)
    ref_o, ref_l = oracle_for(inp, causal=False)
    dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    assert_out_close(out, ref_o, dt, w.name,
                     p_rounding(oracle_for(inp, causal=False, abs_v=True)[0], dt))
    assert_lse_close(lse, ref_l, w.name)
    # The two-kernel decode agrees (the split counts may differ).
    o2, l2 = run_decode(inp)
    assert np.abs(out - o2).max() <= 2e-3 and np.nanmax(np.abs(np.where(np.isinf(l2), 0, lse - l2))) <= 1e-4


def test_decode_fused_config4():
    inp = make_inputs(WORKLOADS["c4_decode_32k"])
    print("[decode fused] c4_decode_32k", flush=True)
    out, lse = run_fused(inp)
    ref_o, ref_l = oracle_for(inp, causal=False)
    assert_out_close(out, ref_o, torch.float16, "c4 fused",
                     p_rounding(oracle_for(inp, causal=False, abs_v=True)[0], torch.float16))
    assert_lse_close(lse, ref_l, "c4 fused")


def test_decode_fused_workspace_reuse():
    """One zeroed workspace serves calls of different shapes in a row; the
    arrival counters are back at zero after each."""
    ws = sa.decode_fused_workspace(3, 40, 40000, 128, "cuda")
    for i, w in enumerate([FUSED_CASES[0], FUSED_CASES[2], FUSED_CASES[3], FUSED_CASES[0], FUSED_CASES[4]]):
        inp = make_inputs(w)
        print(f"[decode fused reuse] call {i}: {w.name}", flush=True)
        out, lse = run_fused(inp, ws)
        assert counters_clear(ws)
        ref_o, ref_l = oracle_for(inp, causal=False)
        dt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
        assert_out_close(out, ref_o, dt, w.name,
                         p_rounding(oracle_for(inp, causal=False, abs_v=True)[0], dt))
        assert_lse_close(lse, ref_l, w.name)


def test_decode_fused_deterministic():
    inp = make_inputs(FUSED_CASES[1])
    a, b = run_fused(inp), run_fused(inp)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


def test_decode_fused_workspace_errors():
    w = FUSED_CASES[0]
    q, k, v, _, _ = to_dev(make_inputs(w))
    small = torch.zeros(128, dtype=torch.uint8, device="cuda")
    with pytest.raises(sa.SaAttnError) as e:
        sa.attn_decode_fused(q, k, v, workspace=small)
    assert e.value.status == sa.SA_ERR_WORKSPACE
