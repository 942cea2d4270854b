"""GPU parity of the prefill kernel (sa_attn_fwd) against the float64 oracle.

Every case draws seeded inputs from ``workloads``, runs the HIP kernel through
the C ABI (via the ctypes binding) and compares element by element with
``oracle.attention`` on the same values: outputs within 5e-3 plus half an ulp of
the output dtype plus the probability-rounding term, lse within 1e-3 (see
tests/parity.py).
"""
import numpy as np
import pytest
import torch

import online_softmax_amd as sa
from parity import assert_lse_close, assert_out_close, oracle_for, p_rounding, to_dev
from workloads import WORKLOADS, Workload, make_inputs, to_f64

pytestmark = pytest.mark.gpu


def run_fwd(inp, causal=None):
    q, k, v, m, s = to_dev(inp)
    w = inp.w
    out, lse = sa.attn_fwd(q, k, v, causal=w.causal if causal is None else causal, scale=w.scale,
                           key_padding_mask=m, alibi_slopes=s)
    torch.cuda.synchronize()
    return to_f64(out.cpu()), lse.cpu().double().numpy()


def check(inp, rows=None, what=""):
    print(f"[fwd] {what or inp.w.name} B={inp.w.B} S_q={inp.w.S_q} S_k={inp.w.S_k} "
          f"H={inp.w.H_q}/{inp.w.H_kv} D={inp.w.D} {inp.w.dtype} causal={inp.w.causal} "
          f"mask={inp.mask is not None} alibi={inp.slopes is not None}", flush=True)
    out, lse = run_fwd(inp)
    ref_o, ref_l = oracle_for(inp, rows=rows)
    if rows is not None:
        out, lse = out[:, rows], lse[:, :, rows]
    dt = torch.float16 if inp.w.dtype == "fp16" else torch.bfloat16
    assert_out_close(out, ref_o, dt, what, p_rounding(oracle_for(inp, rows=rows, abs_v=True)[0], dt))
    assert_lse_close(lse, ref_l, what)
    return out, lse


# Shapes span several 128-row query blocks and 64-key tiles with ragged tails.
SMALL = []
for D in (64, 128):
    for dt in ("fp16", "bf16"):
        for causal in (False, True):
            SMALL.append(Workload(f"s200_D{D}_{dt}_c{int(causal)}", 2, 200, 200, 3, 3, D, dt,
                                  causal=causal, seed=100 + D + causal))


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_plain(w):
    check(make_inputs(w))


FEATURES = [
    Workload("mask_noncausal", 2, 150, 333, 4, 4, 64, "fp16", random_tail=200, seed=11),
    Workload("mask_causal", 2, 333, 333, 4, 4, 128, "bf16", causal=True, random_tail=100, seed=12),
    Workload("alibi_noncausal", 1, 190, 190, 8, 8, 64, "fp16", alibi=True, seed=13),
    Workload("alibi_causal", 1, 260, 260, 8, 8, 128, "bf16", causal=True, alibi=True, seed=14),
    Workload("all_features", 2, 300, 300, 8, 8, 128, "bf16", causal=True, alibi=True, random_tail=64, seed=15),
    Workload("gqa_4to1", 2, 140, 140, 8, 2, 64, "fp16", causal=True, seed=16),
    Workload("gqa_7to1_alibi", 1, 129, 129, 14, 2, 128, "fp16", alibi=True, seed=17),
    Workload("sq_lt_sk_causal", 1, 77, 300, 4, 4, 64, "fp16", causal=True, seed=18),
    Workload("sq_gt_sk_causal", 1, 300, 77, 4, 4, 64, "fp16", causal=True, seed=19),
    Workload("sq_lt_sk_alibi", 1, 50, 200, 4, 4, 128, "bf16", causal=True, alibi=True, seed=20),
    Workload("s1", 3, 1, 1, 2, 2, 64, "fp16", seed=21),
    Workload("s7", 2, 7, 7, 2, 1, 64, "fp16", causal=True, seed=22),
    Workload("s65", 1, 65, 65, 2, 2, 128, "fp16", causal=True, seed=23),
    Workload("s1000", 1, 1000, 1000, 2, 2, 64, "bf16", causal=True, random_tail=300, seed=24),
    Workload("q1_long", 2, 1, 1000, 4, 4, 64, "fp16", seed=25),
    # Causal ALiBi sweeps each workgroup's diagonal band first: rows with no
    # visible key (S_q > S_k) and several band tiles with a ragged end.
    Workload("sq_gt_sk_alibi", 1, 300, 77, 4, 4, 64, "fp16", causal=True, alibi=True, seed=26),
    Workload("s1000_alibi", 1, 1000, 1000, 2, 2, 64, "fp16", causal=True, alibi=True,
             random_tail=300, seed=27),
]


@pytest.mark.parametrize("w", FEATURES, ids=lambda w: w.name)
def test_features(w):
    check(make_inputs(w))


def test_config1_full():
    check(make_inputs(WORKLOADS["c1_fwd_256"]))


def test_config2_full():
    check(make_inputs(WORKLOADS["c2_causal_pad16"]))


def _sample_rows(S, n, seed):
    """Rows at the edges of tiles and blocks plus seeded random ones."""
    base = {0, 1, 63, 64, 127, 128, S // 2, S - 129, S - 128, S - 65, S - 64, S - 2, S - 1}
    rng = np.random.default_rng(seed)
    base |= set(rng.integers(0, S, n).tolist())
    return np.array(sorted(r for r in base if 0 <= r < S))


@pytest.mark.parametrize("name", ["c3_causal_4096", "c3_noncausal_4096"])
def test_config3_sampled(name):
    w = WORKLOADS[name]
    check(make_inputs(w), rows=_sample_rows(w.S_q, 24, 3), what=name)


def test_causal_grid_every_row_written():
    """c3 causal at full size (512 eight-wave workgroups in two groups over
    128-row blocks, issued heaviest first): every row of out and lse is
    written, starting from NaN."""
    w = WORKLOADS["c3_causal_4096"]
    q, k, v, _, _ = to_dev(make_inputs(w))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H_q, w.S_q), float("nan"), dtype=torch.float32, device="cuda")
    sa.attn_fwd(q, k, v, causal=True, scale=w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def test_causal_grid_two_rounds_full():
    """A causal grid of 512 128-row blocks (B * H_q * 4), two per CU on a
    256-CU device, so that the heaviest-first order has a second round to
    fill; checked in full."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    w = Workload("two_round_grid", 2, 512, 512, 64, 8, 64, "fp16", causal=True, seed=131)
    print(f"[fwd] {2 * 64 * 4} blocks on {ncu} CUs", flush=True)
    check(make_inputs(w), what=w.name)


@pytest.mark.parametrize("w", [
    # 192 rows: the second 128-row block sweeps three tiles, so group 1 has
    # none in the last iteration
    Workload("groups_odd_tiles", 1, 192, 192, 4, 4, 128, "fp16", causal=True, seed=141),
    # 100 queries at the end of 1000 keys: 16 tiles, rows skip the last one
    Workload("groups_bottom_right", 2, 100, 1000, 4, 2, 64, "bf16", causal=True, random_tail=300, seed=142),
    # one tile in all (group 1 idle throughout)
    Workload("groups_one_tile", 1, 40, 40, 2, 2, 128, "bf16", causal=True, seed=143),
    Workload("groups_alibi_odd", 1, 192, 192, 4, 4, 128, "bf16", causal=True, alibi=True, random_tail=50,
             seed=144),
    Workload("groups_alibi_bottom_right", 1, 70, 600, 4, 2, 64, "fp16", causal=True, alibi=True, seed=145),
], ids=lambda w: w.name)
def test_two_group_causal(w):
    """Causal shapes that take the two-group forward (eight waves over
    128-row blocks, odd and even tile positions), checked in full; the
    ALiBi cases sweep from the last tile down."""
    check(make_inputs(w), what=w.name)


def test_config5_sampled():
    w = WORKLOADS["c5_alibi_8192"]
    inp = make_inputs(w)
    assert inp.tails == [347, 289]
    check(inp, rows=_sample_rows(w.S_q, 16, 5), what=w.name)


def test_empty_keys():
    """S_k = 0: out = 0 and lse = -inf."""
    q = torch.randn(2, 10, 4, 64, device="cuda").half()
    k = torch.zeros(2, 0, 4, 64, device="cuda").half()
    out, lse = sa.attn_fwd(q, k, k.clone(), causal=False)
    torch.cuda.synchronize()
    assert (out.float() == 0).all() and torch.isneginf(lse).all()


def test_noop_shapes():
    q = torch.zeros(0, 5, 2, 64, device="cuda").half()
    out, lse = sa.attn_fwd(q, q.clone(), q.clone())
    assert out.shape == q.shape and lse.numel() == 0


def test_fully_masked_rows():
    """A batch row whose mask hides every key, and causal rows before the first key."""
    w = Workload("masked_rows", 2, 130, 130, 2, 2, 64, "fp16", causal=True, seed=31)
    inp = make_inputs(w)
    inp.mask = torch.ones((2, 130), dtype=torch.uint8)
    inp.mask[1, :] = 0
    out, lse = check(inp, what="fully masked batch row")
    assert (out[1] == 0).all() and np.isneginf(lse[1]).all()
    # S_q > S_k with causal alignment at the bottom right: early rows see no key.
    w2 = Workload("early_rows", 1, 200, 50, 2, 2, 64, "fp16", causal=True, seed=32)
    out2, lse2 = check(make_inputs(w2), what="rows before the first key")
    assert (out2[0, :150] == 0).all() and np.isneginf(lse2[0, :, :150]).all()


@pytest.mark.parametrize("D,dt", [(128, "bf16"), (64, "fp16")])
def test_alibi_causal_mask_patterns(D, dt):
    """Causal ALiBi with masks other than a tail: the sweep ends at each
    workgroup's last kept key (the tiles after it are cleared throughout), so
    a cleared run followed by kept keys, scattered keys, a long cleared tail
    and a batch row with every key cleared must all match the oracle.

    Batch row 1 keeps only 7 scattered keys, so its rows average at most 7
    values and the probability-rounding term of the bound (parity.p_rounding)
    is what holds it: measured on bf16, 1.04x the bound without that term."""
    w = Workload(f"alibi_mask_patterns_{D}", 4, 700, 700, 4, 2, D, dt, causal=True, alibi=True, seed=33 + D)
    inp = make_inputs(w)
    m = torch.ones((4, 700), dtype=torch.uint8)
    m[0, 100:300] = 0                                      # a cleared run, kept keys after it
    m[1, :] = 0
    m[1, torch.tensor([5, 64, 65, 130, 257, 511, 600])] = 1  # scattered kept keys
    m[2, 41:] = 0                                          # a long cleared tail
    m[3, :] = 0                                            # every key cleared
    inp.mask = m
    print(f"[fwd] {w.name} causal ALiBi, four mask patterns", flush=True)
    out, lse = run_fwd(inp)
    ref_o, ref_l = oracle_for(inp)
    tdt = torch.float16 if dt == "fp16" else torch.bfloat16
    extra = p_rounding(oracle_for(inp, abs_v=True)[0], tdt)
    for b in range(4):
        assert_out_close(out[b], ref_o[b], tdt, f"{w.name} batch row {b}", extra[b])
    assert_lse_close(lse, ref_l, w.name)
    assert (out[3] == 0).all() and np.isneginf(lse[3]).all()
    assert np.isneginf(lse[2, :, :41]).sum() == 0


def test_single_key_bitwise():
    """S_k = 1: P = 1 exactly, so out equals v bit for bit."""
    w = Workload("one_key", 2, 100, 1, 4, 2, 128, "bf16", seed=33)
    inp = make_inputs(w)
    out, lse = check(inp)
    v = to_f64(inp.v)
    for h in range(4):
        assert (out[:, :, h, :] == v[:, 0:1, h // 2, :]).all()


def test_overflow_guard():
    """q.k far past the fp16 range stays finite with float32 scores.

    Scores here reach about 1e4, where one float32 ulp of the accumulated dot
    product is already about 1e-3; the lse bound is therefore the 1e-3 budget
    plus the float32 dot-product error bound 2 D u scale max_j sum_d |q_d k_jd|
    (u = 2^-24).  Outputs keep the usual bound.
    """
    w = Workload("big_values", 1, 100, 100, 2, 2, 64, "fp16", causal=True, seed=34)
    inp = make_inputs(w, scale_qk=64.0)
    out, lse = run_fwd(inp)
    ref_o, ref_l = oracle_for(inp)
    assert np.abs(np.einsum("bihd,bjhd->bhij", to_f64(inp.q), to_f64(inp.k))).max() > 65504
    assert_out_close(out, ref_o, torch.float16, "large magnitudes",
                     p_rounding(oracle_for(inp, abs_v=True)[0], torch.float16))
    q, k = to_f64(inp.q), to_f64(inp.k)
    mag = np.einsum("bihd,bjhd->bhij", np.abs(q), np.abs(k)).max(axis=-1)  # [B, H, S_q]
    bound = 1e-3 + 2 * w.D * 2.0 ** -24 * w.scale * mag
    assert np.isfinite(lse).all()
    assert (np.abs(lse - ref_l) <= bound).all(), np.abs(lse - ref_l).max()


def test_deterministic():
    """Two runs of the same call are bitwise identical."""
    inp = make_inputs(Workload("det", 2, 300, 300, 4, 4, 128, "bf16", causal=True, alibi=True,
                               random_tail=50, seed=35))
    a = run_fwd(inp)
    b = run_fwd(inp)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()


def test_causal_leak_bitwise():
    """Changing keys/values no row may see leaves out and lse bit-identical."""
    w = Workload("leak", 1, 256, 256, 4, 4, 64, "fp16", causal=True, pad_tail=40, seed=36)
    inp = make_inputs(w)
    a = run_fwd(inp)
    g = torch.Generator().manual_seed(99)
    k2, v2 = inp.k.clone(), inp.v.clone()
    # Perturb the padded keys (hidden from every row).
    k2[:, -40:] = torch.randn(k2[:, -40:].shape, generator=g).half()
    v2[:, -40:] = torch.randn(v2[:, -40:].shape, generator=g).half()
    inp2 = make_inputs(w)
    inp2.k, inp2.v = k2, v2
    b = run_fwd(inp2)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
    # Perturb keys after position 100: rows 0..100 must not change.
    k3, v3 = inp.k.clone(), inp.v.clone()
    k3[:, 101:] = torch.randn(k3[:, 101:].shape, generator=g).half()
    v3[:, 101:] = torch.randn(v3[:, 101:].shape, generator=g).half()
    inp3 = make_inputs(w)
    inp3.k, inp3.v = k3, v3
    c = run_fwd(inp3)
    assert (a[0][:, :101] == c[0][:, :101]).all() and (a[1][:, :, :101] == c[1][:, :, :101]).all()


def _eight_wave(w):
    """Whether the forward of this shape runs 256-row eight-wave workgroups
    (one group): enough of them for every CU, four per CU when causal."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    return w.B * w.H_q * -(-w.S_q // 256) >= ncu * (4 if w.causal else 1)


EIGHT_WAVE = [
    # causal: B * H_q * ceil(S_q / 256) = 1024 workgroups (four per CU on 256 CUs)
    Workload("w8_causal_f16_d128", 4, 300, 300, 128, 32, 128, "fp16", causal=True, seed=150),
    Workload("w8_causal_mask_bf16_d64", 4, 300, 300, 128, 128, 64, "bf16", causal=True, random_tail=90,
             seed=151),
    Workload("w8_causal_alibi_f16_d64", 4, 300, 300, 128, 16, 64, "fp16", causal=True, alibi=True, seed=152),
    Workload("w8_causal_all_f16_d128", 4, 300, 300, 128, 64, 128, "fp16", causal=True, alibi=True,
             random_tail=70, seed=153),
    Workload("w8_causal_all_bf16_d128", 4, 300, 300, 128, 128, 128, "bf16", causal=True, alibi=True,
             random_tail=130, seed=154),
    # non-causal: 2 * 64 * 2 = 256 workgroups
    Workload("w8_plain_f16_d64", 2, 300, 300, 64, 8, 64, "fp16", seed=155),
    Workload("w8_all_bf16_d128", 2, 300, 333, 64, 64, 128, "bf16", alibi=True, random_tail=100, seed=156),
    Workload("w8_mask_f16_d128_sq_lt_sk", 2, 280, 500, 64, 16, 128, "fp16", random_tail=200, seed=157),
]


def _persistent_units(w):
    """Units of the forward's persistent schedule for this shape (a causal
    unit pairs two query blocks) and whether it takes it: eight-wave
    workgroups (256-row blocks, or 128-row blocks in two groups under the
    causal rule) and at least two units per CU."""
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    nw = 8 if _eight_wave(w) else 4
    if nw == 4 and not w.causal:
        return 0, False
    nmb = -(-w.S_q // (32 * nw))
    units = w.B * w.H_q * (-(-nmb // 2) if w.causal else nmb)
    return units, units >= 2 * ncu


PERSISTENT = [
    # 256-row blocks without the causal rule: 512 units of one block
    Workload("persist_plain_f16_d64", 2, 300, 300, 128, 16, 64, "fp16", seed=160),
    # 128-row blocks in two groups, five per head: units of blocks 4 and 0,
    # 3 and 1, and block 2 alone
    Workload("persist_groups_odd_f16_d64", 4, 640, 640, 64, 16, 64, "fp16", causal=True, random_tail=100,
             seed=161),
    Workload("persist_groups_alibi_bf16_d64", 4, 600, 640, 64, 8, 64, "bf16", causal=True, alibi=True, seed=162),
    # 256-row blocks under the causal rule with ALiBi and padding (the c5
    # layout): units of blocks 3 and 0, 2 and 1; the second block of each
    # unit sweeps from its last tile down
    Workload("persist_w8_alibi_mask_bf16_d64", 4, 1024, 1024, 64, 64, 64, "bf16", causal=True, alibi=True,
             random_tail=300, seed=164),
]


@pytest.mark.parametrize("w", PERSISTENT, ids=lambda w: w.name)
def test_persistent_schedule_full(w):
    """Shapes with at least two units per CU, where each workgroup of the
    forward works through a list of (batch, head, block pair) units: checked
    in full against the oracle."""
    units, persistent = _persistent_units(w)
    print(f"[fwd] {w.name}: {units} units, persistent schedule: {persistent}", flush=True)
    if not persistent:
        pytest.skip("this device has too many compute units for the shape to take the persistent schedule")
    check(make_inputs(w), what=w.name)


def test_persistent_schedule_ragged_units_sampled():
    """600 units (eight-wave causal pairs; 150 heads of 1800 rows) spread
    unevenly over the XCDs and CUs: sampled rows, and every row written."""
    w = Workload("persist_ragged_units", 3, 1800, 1800, 50, 10, 64, "fp16", causal=True, random_tail=200, seed=163)
    units, persistent = _persistent_units(w)
    print(f"[fwd] {w.name}: {units} units, persistent schedule: {persistent}", flush=True)
    if not persistent:
        pytest.skip("this device has too many compute units for the shape to take the persistent schedule")
    inp = make_inputs(w)
    out, lse = check(inp, rows=_sample_rows(w.S_q, 16, 7), what=w.name)
    q, k, v, m, s = to_dev(inp)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((w.B, w.H_q, w.S_q), float("nan"), dtype=torch.float32, device="cuda")
    sa.attn_fwd(q, k, v, causal=True, scale=w.scale, key_padding_mask=m, out=o2, lse=l2)
    torch.cuda.synchronize()
    assert not torch.isnan(o2).any() and not torch.isnan(l2).any()


@pytest.mark.parametrize("w", EIGHT_WAVE, ids=lambda w: w.name)
def test_eight_wave_full(w):
    """Grids large enough for the 256-row eight-wave workgroups, checked in
    full: every rule (causal, padding, ALiBi) on D = 64 and 128, fp16 and bf16,
    with ragged ends (300 rows: a full block and a part block)."""
    if not _eight_wave(w):
        pytest.skip("this device has too many compute units for the shape to take eight waves")
    check(make_inputs(w), what=w.name)


@pytest.mark.parametrize("w", [
    Workload("constv_causal_alibi_bf16", 2, 300, 300, 4, 2, 128, "bf16", causal=True, alibi=True,
             random_tail=60, seed=160),
    Workload("constv_plain_f16", 1, 257, 700, 8, 8, 64, "fp16", seed=161),
    Workload("constv_w8_causal_bf16", 4, 300, 300, 128, 32, 128, "bf16", causal=True, alibi=True, seed=162),
], ids=lambda w: w.name)
def test_constant_v(w):
    """Constant values (every v_j = c): the output is c on every row that
    sees a key, 0 on the others (pin of the weights' normalisation).  The row
    sum takes the unrounded probabilities and P.V the rounded ones, so out =
    c * sum(rounded) / sum(unrounded): within the plain bound plus the
    probability-rounding term u |c| (parity.p_rounding)."""
    inp = make_inputs(w)
    c = torch.zeros_like(inp.v)
    c[..., :] = torch.linspace(-3.0, 3.0, w.D).to(inp.v.dtype)  # one value per column
    inp.v = c
    out, lse = run_fwd(inp)
    ref_o, ref_l = oracle_for(inp)
    rows = np.isfinite(ref_l).transpose(0, 2, 1)                 # [B, S_q, H]
    want = np.where(rows[..., None], to_f64(c[:, :1]).repeat(w.H_q // w.H_kv, axis=2), 0.0)
    assert np.abs(ref_o - want).max() <= 1e-12                   # the oracle itself
    tdt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    print(f"[fwd] {w.name}: constant values, {int(rows.sum())} rows with keys", flush=True)
    assert_out_close(out, want, tdt, w.name, p_rounding(np.abs(want), tdt))
    assert (out[~rows] == 0).all()
    assert_lse_close(lse, ref_l, w.name)


def test_config5_every_element_finite():
    """The c5 shape ([2, 8192, 32, 128] bf16, causal, ALiBi, padding tails):
    every element of out and lse is finite (no NaN or Inf up to S = 8192),
    checked on the device over the whole output, which starts as NaN."""
    w = WORKLOADS["c5_alibi_8192"]
    q, k, v, m, s = to_dev(make_inputs(w))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H_q, w.S_q), float("nan"), dtype=torch.float32, device="cuda")
    sa.attn_fwd(q, k, v, causal=True, scale=w.scale, key_padding_mask=m, alibi_slopes=s, out=out, lse=lse)
    torch.cuda.synchronize()
    print(f"[fwd] {w.name}: finite sweep over {out.numel()} outputs and {lse.numel()} lse", flush=True)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all())
