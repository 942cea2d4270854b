"""Host-side tests of libsa_attn (no GPU needed).

The library is loaded with ctypes; every function the public header declares
must be exported with the signature the binding uses.  Argument validation
runs before any HIP call, so invalid requests (null or misaligned pointers,
bad sizes, unsupported D or dtype, short workspace, overlapping buffers) are
checked here with fake addresses that are never dereferenced.  No call in this
file reaches a kernel launch.
"""
import ctypes
import re
from pathlib import Path

import pytest

import online_softmax_amd as sa

HEADER = Path(__file__).resolve().parents[1] / "include" / "sa_attn.h"


@pytest.fixture(scope="module")
def L():
    if not sa.LIB_PATH.exists():
        from online_softmax_amd.build import build
        build()
    return sa.lib()


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(L):
    names = declared_functions()
    assert names == sorted(sa.SIGNATURES), names
    for n in names:
        assert hasattr(L, n), f"{n} is declared in sa_attn.h but not exported"


# Fake, 256-byte aligned, non-overlapping addresses (never dereferenced).
A = 1 << 40
Q, K, V, O, LSE, WS, SL = (A + i * (1 << 32) for i in range(7))


def fwd(L, q=Q, k=K, v=V, out=O, lse=LSE, B=1, S_q=8, S_k=8, H_q=2, H_kv=2, D=64, scale=0.125,
        causal=0, mask=None, slopes=None, dtype=0):
    return L.sa_attn_fwd(q, k, v, out, lse, B, S_q, S_k, H_q, H_kv, D, scale, causal, mask, slopes,
                         dtype, None)


def dec(L, q=Q, k=K, v=V, out=O, lse=LSE, B=1, S_k=100, H_q=4, H_kv=2, D=64, scale=0.125,
        mask=None, slopes=None, dtype=0, ws=WS, wsb=None):
    if wsb is None:
        wsb = L.sa_attn_decode_workspace_size(B, H_q, S_k, D)
    return L.sa_attn_decode(q, k, v, out, lse, B, S_k, H_q, H_kv, D, scale, mask, slopes, dtype,
                            ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), sa.SA_ERR_INVALID_ARG),
    (dict(out=None), sa.SA_ERR_INVALID_ARG),
    (dict(k=None), sa.SA_ERR_INVALID_ARG),
    (dict(q=Q + 8), sa.SA_ERR_INVALID_ARG),
    (dict(lse=LSE + 2), sa.SA_ERR_INVALID_ARG),
    (dict(D=96), sa.SA_ERR_UNSUPPORTED),
    (dict(D=256), sa.SA_ERR_UNSUPPORTED),
    (dict(dtype=2), sa.SA_ERR_UNSUPPORTED),
    (dict(H_q=3, H_kv=2), sa.SA_ERR_INVALID_ARG),
    (dict(H_kv=0), sa.SA_ERR_INVALID_ARG),
    (dict(S_q=-1), sa.SA_ERR_INVALID_ARG),
    (dict(S_k=-5), sa.SA_ERR_INVALID_ARG),
    (dict(causal=2), sa.SA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), sa.SA_ERR_INVALID_ARG),
    (dict(out=Q), sa.SA_ERR_INVALID_ARG),          # out aliases q
    (dict(lse=K + 16), sa.SA_ERR_INVALID_ARG),     # lse inside k
    (dict(slopes=SL, scale=0.0), sa.SA_ERR_INVALID_ARG),  # ALiBi needs a nonzero scale
])
def test_fwd_rejects(L, kw, code):
    assert fwd(L, **kw) == code
    assert sa.last_error() != ""


def test_fwd_noop_needs_no_pointers(L):
    assert fwd(L, q=None, out=None, k=None, v=None, B=0) == sa.SA_OK
    assert fwd(L, q=None, out=None, k=None, v=None, S_q=0) == sa.SA_OK
    assert sa.last_error() == ""


@pytest.mark.parametrize("kw,code", [
    (dict(ws=None), sa.SA_ERR_WORKSPACE),
    (dict(wsb=16), sa.SA_ERR_WORKSPACE),
    (dict(ws=WS + 4), sa.SA_ERR_WORKSPACE),
    (dict(v=None), sa.SA_ERR_INVALID_ARG),
    (dict(D=32), sa.SA_ERR_UNSUPPORTED),
    (dict(dtype=-1), sa.SA_ERR_UNSUPPORTED),
    (dict(H_q=6, H_kv=4), sa.SA_ERR_INVALID_ARG),
    (dict(ws=K), sa.SA_ERR_INVALID_ARG),           # workspace overlaps k_cache
    (dict(out=WS), sa.SA_ERR_INVALID_ARG),         # out inside the workspace
    (dict(slopes=SL, scale=0.0), sa.SA_ERR_INVALID_ARG),  # ALiBi needs a nonzero scale
])
def test_decode_rejects(L, kw, code):
    assert dec(L, **kw) == code


def test_decode_noop(L):
    assert dec(L, B=0, q=None, out=None, ws=None, wsb=0) == sa.SA_OK


def test_status_strings(L):
    for code, name in [(0, "SA_OK"), (1, "SA_ERR_INVALID_ARG"), (2, "SA_ERR_UNSUPPORTED"),
                       (3, "SA_ERR_WORKSPACE"), (4, "SA_ERR_HIP")]:
        assert sa.status_string(code) == name
    assert "unknown" in sa.status_string(99)


def test_decode_splits_and_workspace(L):
    # 32K keys, 4 sequences, 14:2 GQA on 256 CUs: 8 (batch, KV head) pairs,
    # one workgroup per CU -> 32 splits of 1024 keys.
    assert sa.decode_num_splits(4, 32768, 14, 2, 256) == 32
    assert sa.decode_num_splits(4, 32768, 14, 2, 304) == 37  # 38 -> 863 -> 896 keys
    # Batch 1: 2 pairs -> 128 splits of 256 keys; the single-kernel decode
    # caps them at 64 (512 keys), and takes the same count where it is lower.
    assert sa.decode_num_splits(1, 32768, 14, 2, 256) == 128
    assert sa.decode_fused_num_splits(1, 32768, 14, 2, 256) == 64
    assert sa.decode_fused_num_splits(4, 32768, 14, 2, 256) == 32
    # 40000 keys over at most 64 splits: 625 -> 640-key splits, 63 of them.
    assert sa.decode_fused_num_splits(1, 40000, 32, 2, 256) == 63
    # Never more splits than 128-key steps, never fewer than one.
    assert sa.decode_num_splits(1, 100, 8, 8, 256) == 1
    assert sa.decode_num_splits(1, 1000, 1, 1, 256) == 8
    assert sa.decode_num_splits(1, 10 ** 7, 1, 1, 256) == 256
    assert sa.decode_num_splits(64, 32768, 64, 8, 256) == 1
    # One (batch, KV head, head group): 256 splits of 128 keys.
    assert sa.decode_num_splits(1, 32768, 4, 1, 256) == 256
    for B, Hq, Hkv, S in [(4, 14, 2, 32768), (1, 40, 1, 300), (3, 8, 8, 1), (2, 6, 3, 129),
                          (1, 4, 1, 32768)]:
        n = sa.decode_num_splits(B, S, Hq, Hkv, 256)
        # Partial outputs and partial lse of every split.
        need = B * Hq * n * (64 + 1) * 4
        assert sa.decode_workspace_size(B, Hq, S, 64) >= need
    assert sa.decode_workspace_size(-1, 1, 1, 64) == 0
    assert sa.decode_workspace_size(0, 1, 1, 64) >= 0
    # The single-kernel decode: 64 KiB of arrival counters, then the same area.
    L = sa.lib()
    for B, Hq, S, D in [(4, 14, 32768, 64), (1, 40, 300, 128), (0, 8, 1, 64)]:
        assert L.sa_attn_decode_fused_workspace_size(B, Hq, S, D) == \
            sa.DECODE_ARRIVE_BYTES + sa.decode_workspace_size(B, Hq, S, D)
    assert L.sa_attn_decode_fused_workspace_size(-1, 1, 1, 64) == 0


# Backward: more fake buffers beside the forward's.
DO, DQ, DK, DV = (A + i * (1 << 32) for i in range(7, 11))


def bwd(L, q=Q, k=K, v=V, out=O, dout=DO, lse=LSE, dq=DQ, dk=DK, dv=DV, B=1, S_q=8, S_k=8, H_q=2,
        H_kv=2, D=64, scale=0.125, causal=0, mask=None, slopes=None, dtype=0, ws=WS, wsb=None):
    if wsb is None:
        wsb = L.sa_attn_bwd_workspace_size(B, H_q, S_q)
    return L.sa_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, S_q, S_k, H_q, H_kv, D, scale,
                         causal, mask, slopes, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), sa.SA_ERR_INVALID_ARG),
    (dict(dq=None), sa.SA_ERR_INVALID_ARG),
    (dict(dv=None), sa.SA_ERR_INVALID_ARG),
    (dict(lse=None), sa.SA_ERR_INVALID_ARG),
    (dict(dk=DK + 8), sa.SA_ERR_INVALID_ARG),      # misaligned
    (dict(lse=LSE + 2), sa.SA_ERR_INVALID_ARG),
    (dict(D=96), sa.SA_ERR_UNSUPPORTED),
    (dict(dtype=3), sa.SA_ERR_UNSUPPORTED),
    (dict(H_q=5, H_kv=2), sa.SA_ERR_INVALID_ARG),
    (dict(S_q=-1), sa.SA_ERR_INVALID_ARG),
    (dict(causal=-1), sa.SA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), sa.SA_ERR_INVALID_ARG),
    (dict(slopes=SL, scale=0.0), sa.SA_ERR_INVALID_ARG),
    (dict(ws=None), sa.SA_ERR_WORKSPACE),
    (dict(wsb=8), sa.SA_ERR_WORKSPACE),
    (dict(ws=WS + 8), sa.SA_ERR_WORKSPACE),
    (dict(dq=Q), sa.SA_ERR_INVALID_ARG),           # dq aliases q
    (dict(dk=DO + 64), sa.SA_ERR_INVALID_ARG),     # dk inside dout
    (dict(dv=DK), sa.SA_ERR_INVALID_ARG),          # dv aliases dk
    (dict(ws=DQ), sa.SA_ERR_INVALID_ARG),          # workspace aliases dq
])
def test_bwd_rejects(L, kw, code):
    assert bwd(L, **kw) == code
    assert sa.last_error() != ""


def test_bwd_noop_and_workspace(L):
    assert bwd(L, B=0, q=None, dq=None, ws=None, wsb=0) == sa.SA_OK
    assert bwd(L, S_q=0, S_k=0, q=None, k=None, dq=None, dk=None, ws=None, wsb=0) == sa.SA_OK
    # One {lse2, Di} float pair per query row.
    assert sa.bwd_workspace_size(2, 14, 4096) == 2 * 14 * 4096 * 8
    assert sa.bwd_workspace_size(-1, 1, 1) == 0


BIAS = A + 11 * (1 << 32)


def ext(L, q=Q, k=K, v=V, out=O, lse=LSE, B=1, S_q=8, S_k=8, H_q=2, H_kv=2, D=64, scale=0.125,
        causal=0, mask=None, slopes=None, bias=BIAS, sb=0, sh=0, sq=8, p=0.0, dtype=0):
    return L.sa_attn_fwd_ext(q, k, v, out, lse, B, S_q, S_k, H_q, H_kv, D, scale, causal, mask,
                             slopes, bias, sb, sh, sq, p, 0, 0, dtype, None)


@pytest.mark.parametrize("kw", [
    dict(scale=0.0),                    # a bias is added in units of 1/|scale|
    dict(scale=-0.0),
    dict(scale=1e-45),                  # 1/|scale| overflows float32
    dict(bias=None, slopes=SL, scale=0.0),
    dict(bias=None, slopes=SL, scale=1e-45),
    dict(p=1.0),
    dict(sq=6),                         # stride not a multiple of 4
    dict(bias=BIAS + 4),                # misaligned bias
    dict(out=BIAS),                     # out overlaps the bias
])
def test_ext_rejects(L, kw):
    assert ext(L, **kw) == sa.SA_ERR_INVALID_ARG
    assert sa.last_error() != ""


def test_bias_scale_rule(L):
    """With no bias, a zero scale is valid (every score is 0); with one, the
    tiniest normal scale still has a finite 1/|scale|, so validation passes up
    to the launch step (no call here reaches a launch: B = 0 stops it after
    the argument checks)."""
    assert ext(L, bias=None, scale=0.0, B=0) == sa.SA_OK
    assert fwd(L, slopes=SL, scale=1e-45) == sa.SA_ERR_INVALID_ARG
    assert dec(L, slopes=SL, scale=1e-45) == sa.SA_ERR_INVALID_ARG
    assert "1/|scale|" in sa.last_error()


def test_decode_noalloc_argument_checks(L):
    """The allocation-free decode checks its arguments before any HIP call."""
    def call(q=Q, k=K, v=V, out=O, lse=LSE, B=1, S_k=100, H_q=4, H_kv=2, D=64, scale=0.125, dtype=0):
        return L.sa_attn_decode_noalloc(q, k, v, out, lse, B, S_k, H_q, H_kv, D, scale, None, None, dtype, None)
    assert call(B=0, q=None, out=None) == sa.SA_OK
    assert call(q=None) == sa.SA_ERR_INVALID_ARG
    assert call(out=Q) == sa.SA_ERR_INVALID_ARG
    assert call(D=96) == sa.SA_ERR_UNSUPPORTED
    assert call(H_q=5) == sa.SA_ERR_INVALID_ARG
