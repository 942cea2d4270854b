"""Streaming exact attention (online softmax) for AMD MI355X — Python binding.

A thin ctypes layer over ``libsa_attn.so`` (C ABI declared in
``include/sa_attn.h``).  It only marshals arguments: it checks tensor
devices, dtypes, shapes and contiguity, passes raw device pointers and the
current HIP stream, and raises on a non-OK status.  All arithmetic runs in the
library's HIP kernels; there is no CPU or PyTorch fallback, and every call
raises if the library was not built.

Functions keep the names of the C entry points:

* ``attn_fwd(q, k, v, causal=False, scale=None, key_padding_mask=None,
  alibi_slopes=None, out=None, lse=None, return_lse=True)``
* ``attn_decode(q, k_cache, v_cache, scale=None, key_padding_mask=None,
  alibi_slopes=None, out=None, lse=None, workspace=None, return_lse=True)``
* ``decode_workspace_size(B, H_q, S_k, D)`` and ``decode_num_splits(...)``
* ``attn_decode_noalloc(...)`` (no workspace: the library's own scratch)
* ``attn_decode_fused(...)`` (one kernel) and
  ``decode_fused_workspace(B, H_q, S_k, D, device)``
* ``attn_fwd_block_sparse(q, k, v, block_mask, causal=False, ...)``
* ``attn_fwd_ext(q, k, v, causal=False, ..., attn_bias=None, dropout_p=0.0,
  seed=0, offset=0)``
* ``attn_bwd(q, k, v, out, dout, lse, causal=False, scale=None, key_padding_mask=None,
  alibi_slopes=None)`` -> ``(dq, dk, dv)`` and ``bwd_workspace_size(B, H_q, S_q)``
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path
from typing import Optional

import torch

LIB_PATH = Path(__file__).resolve().parent / "libsa_attn.so"

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)
SA_F16, SA_BF16 = 0, 1
_DTYPE = {torch.float16: SA_F16, torch.bfloat16: SA_BF16}

# Every symbol the public header declares, with its ctypes signature.
_VP, _FP, _U8P = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
_I, _F, _SZ = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_I64, _D, _U64, _U32 = ctypes.c_int64, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32
SIGNATURES = {
    "sa_attn_fwd": (_I, [_VP, _VP, _VP, _VP, _FP, _I, _I, _I, _I, _I, _I, _F, _I, _U8P, _FP, _I, _VP]),
    "sa_attn_fwd_block_sparse": (_I, [_VP, _VP, _VP, _VP, _FP, _I, _I, _I, _I, _I, _I, _F, _I, _U8P, _FP,
                                      _U8P, _I, _VP]),
    "sa_attn_fwd_ext": (_I, [_VP, _VP, _VP, _VP, _FP, _I, _I, _I, _I, _I, _I, _F, _I, _U8P, _FP,
                             _FP, _I64, _I64, _I64, _D, _U64, _U32, _I, _VP]),
    "sa_attn_decode_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "sa_attn_decode": (_I, [_VP, _VP, _VP, _VP, _FP, _I, _I, _I, _I, _I, _F, _U8P, _FP, _I, _VP, _SZ, _VP]),
    "sa_attn_decode_noalloc": (_I, [_VP, _VP, _VP, _VP, _FP, _I, _I, _I, _I, _I, _F, _U8P, _FP, _I, _VP]),
    "sa_attn_decode_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "sa_attn_decode_fused_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "sa_attn_decode_fused_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "sa_attn_decode_fused": (_I, [_VP, _VP, _VP, _VP, _FP, _I, _I, _I, _I, _I, _F, _U8P, _FP, _I, _VP, _SZ, _VP]),
    "sa_attn_bwd_workspace_size": (_SZ, [_I, _I, _I]),
    "sa_attn_bwd": (_I, [_VP, _VP, _VP, _VP, _VP, _FP, _VP, _VP, _VP, _I, _I, _I, _I, _I, _I, _F,
                         _I, _U8P, _FP, _I, _VP, _SZ, _VP]),
    "sa_status_string": (ctypes.c_char_p, [_I]),
    "sa_last_error": (ctypes.c_char_p, []),
}

_lib: Optional[ctypes.CDLL] = None


class SaAttnError(RuntimeError):
    """A non-OK status from libsa_attn."""

    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{status_string(status)}: {detail}")


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m online_softmax_amd.build` "
                               "(there is no fallback implementation)")
        h = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().sa_status_string(status).decode()


def last_error() -> str:
    return lib().sa_last_error().decode()


def _check(status: int) -> None:
    if status != SA_OK:
        raise SaAttnError(status, last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _mask_arg(mask, B, S_k, dev):
    if mask is None:
        return None
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    _need(mask, "key_padding_mask", torch.uint8, (B, S_k), dev)
    return mask


def _fwd_prepare(q, k, v, key_padding_mask, alibi_slopes, out, lse, return_lse, scale):
    """Checks and output allocation shared by the two forwards."""
    _need(q, "q")
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    B, S_q, H_q, D = q.shape
    _need(k, "k", q.dtype, None, dev)
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k has shape {tuple(k.shape)}, incompatible with q {tuple(q.shape)}")
    S_k, H_kv = k.shape[1], k.shape[2]
    _need(v, "v", q.dtype, k.shape, dev)
    mask = _mask_arg(key_padding_mask, B, S_k, dev)
    if alibi_slopes is not None:
        _need(alibi_slopes, "alibi_slopes", torch.float32, (H_q,), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H_q, S_q), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H_q, S_q), dev)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return dev, (B, S_q, S_k, H_q, H_kv, D), mask, out, lse, sc


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
             scale: Optional[float] = None, key_padding_mask: Optional[torch.Tensor] = None,
             alibi_slopes: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, return_lse: bool = True):
    """Attention forward through ``sa_attn_fwd``.

    q ``[B, S_q, H_q, D]``, k/v ``[B, S_k, H_kv, D]`` (fp16 or bf16, same
    device); key_padding_mask ``[B, S_k]`` bool/uint8 (nonzero keeps);
    alibi_slopes float32 ``[H_q]``.  Returns ``out`` (and float32 ``lse``
    ``[B, H_q, S_q]`` when ``return_lse``).
    """
    dev, (B, S_q, S_k, H_q, H_kv, D), mask, out, lse, sc = _fwd_prepare(
        q, k, v, key_padding_mask, alibi_slopes, out, lse, return_lse, scale)
    st = lib().sa_attn_fwd(q.data_ptr(), _ptr(k), _ptr(v), out.data_ptr(), _ptr(lse),
                           B, S_q, S_k, H_q, H_kv, D, sc, int(bool(causal)), _ptr(mask),
                           _ptr(alibi_slopes), _DTYPE[q.dtype], _stream(dev))
    _check(st)
    return (out, lse) if return_lse else out


SPARSE_BLOCK = 128  # query rows and keys per block of the block-sparse forward
DECODE_ARRIVE_BYTES = 65536  # arrival counters at the start of a single-kernel decode workspace


def attn_fwd_block_sparse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          block_mask: torch.Tensor, causal: bool = False,
                          scale: Optional[float] = None,
                          key_padding_mask: Optional[torch.Tensor] = None,
                          alibi_slopes: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          return_lse: bool = True):
    """Block-sparse attention forward through ``sa_attn_fwd_block_sparse``.

    As ``attn_fwd``, with ``block_mask`` bool/uint8
    ``[B, H_q, ceil(S_q / 128), ceil(S_k / 128)]`` (nonzero = the query block
    attends to the key block).
    """
    dev, (B, S_q, S_k, H_q, H_kv, D), mask, out, lse, sc = _fwd_prepare(
        q, k, v, key_padding_mask, alibi_slopes, out, lse, return_lse, scale)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    nbq, nbk = -(-S_q // SPARSE_BLOCK), -(-S_k // SPARSE_BLOCK)
    _need(block_mask, "block_mask", torch.uint8, (B, H_q, nbq, nbk), dev)
    st = lib().sa_attn_fwd_block_sparse(q.data_ptr(), _ptr(k), _ptr(v), out.data_ptr(), _ptr(lse),
                                        B, S_q, S_k, H_q, H_kv, D, sc, int(bool(causal)),
                                        _ptr(mask), _ptr(alibi_slopes), block_mask.data_ptr(),
                                        _DTYPE[q.dtype], _stream(dev))
    _check(st)
    return (out, lse) if return_lse else out


def attn_fwd_ext(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                 scale: Optional[float] = None, key_padding_mask: Optional[torch.Tensor] = None,
                 alibi_slopes: Optional[torch.Tensor] = None,
                 attn_bias: Optional[torch.Tensor] = None, dropout_p: float = 0.0, seed: int = 0,
                 offset: int = 0, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, return_lse: bool = True):
    """Forward with an additive float mask and dropout through ``sa_attn_fwd_ext``.

    As ``attn_fwd``, plus ``attn_bias``: a float32 tensor on the same device,
    broadcastable to ``[B, H_q, S_q, S_k]`` (-inf hides a key); and dropout
    with probability ``dropout_p``, 64-bit ``seed`` and 32-bit ``offset``.
    A bias whose row strides are not multiples of 4 elements (or whose key
    axis is not contiguous) is copied into a padded buffer first.
    """
    dev, (B, S_q, S_k, H_q, H_kv, D), mask, out, lse, sc = _fwd_prepare(
        q, k, v, key_padding_mask, alibi_slopes, out, lse, return_lse, scale)
    bias, strides = None, (0, 0, 0)
    if attn_bias is not None:
        if not isinstance(attn_bias, torch.Tensor) or attn_bias.dtype != torch.float32:
            raise ValueError("attn_bias must be a float32 tensor")
        if attn_bias.device != dev:
            raise ValueError(f"attn_bias is on {attn_bias.device}, expected {dev}")
        try:
            bias = attn_bias.expand(B, H_q, S_q, S_k)
        except RuntimeError as e:
            raise ValueError(f"attn_bias of shape {tuple(attn_bias.shape)} does not broadcast to "
                             f"{(B, H_q, S_q, S_k)}") from e
        st4 = bias.stride()
        if S_k > 1 and st4[3] != 1 or any(x % 4 for x in st4[:3]) or bias.data_ptr() % 16:
            # Pad the key axis to a multiple of 4 in a fresh buffer (axes the
            # caller broadcast stay broadcast).
            shape = [n if attn_bias.dim() - 4 + ax >= 0 and attn_bias.shape[attn_bias.dim() - 4 + ax] != 1
                     else 1 for ax, n in enumerate((B, H_q, S_q, S_k))]
            shape[3] = S_k
            padded = torch.empty(shape[:3] + [-(-S_k // 4) * 4], dtype=torch.float32, device=dev)
            padded[..., :S_k] = attn_bias.expand(*shape)
            bias = padded[..., :S_k].expand(B, H_q, S_q, S_k)
            st4 = bias.stride()
        strides = st4[:3]
    st = lib().sa_attn_fwd_ext(q.data_ptr(), _ptr(k), _ptr(v), out.data_ptr(), _ptr(lse),
                               B, S_q, S_k, H_q, H_kv, D, sc, int(bool(causal)), _ptr(mask),
                               _ptr(alibi_slopes), None if bias is None else bias.data_ptr(),
                               strides[0], strides[1], strides[2], float(dropout_p),
                               int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 32 - 1),
                               _DTYPE[q.dtype], _stream(dev))
    _check(st)
    return (out, lse) if return_lse else out


def decode_workspace_size(B: int, H_q: int, S_k: int, D: int) -> int:
    return int(lib().sa_attn_decode_workspace_size(B, H_q, S_k, D))


def decode_num_splits(B: int, S_k: int, H_q: int, H_kv: int, num_cu: int) -> int:
    return int(lib().sa_attn_decode_num_splits(B, S_k, H_q, H_kv, num_cu))


def decode_fused_num_splits(B: int, S_k: int, H_q: int, H_kv: int, num_cu: int) -> int:
    return int(lib().sa_attn_decode_fused_num_splits(B, S_k, H_q, H_kv, num_cu))


def decode_workspace(B: int, H_q: int, S_k: int, D: int, device) -> torch.Tensor:
    """A device byte buffer large enough for ``attn_decode`` at these sizes
    (reusable by calls issued one after another on a stream)."""
    n = decode_workspace_size(B, H_q, S_k, D)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _decode_prepare(q, k_cache, v_cache, key_padding_mask, alibi_slopes, out, lse, return_lse, scale):
    """Checks and output allocation shared by the two decodes."""
    _need(q, "q")
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    B, one, H_q, D = q.shape
    if one != 1:
        raise ValueError("decode takes exactly one query token per sequence")
    _need(k_cache, "k_cache", q.dtype, None, dev)
    if k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError(f"k_cache has shape {tuple(k_cache.shape)}, incompatible with q")
    S_k, H_kv = k_cache.shape[1], k_cache.shape[2]
    _need(v_cache, "v_cache", q.dtype, k_cache.shape, dev)
    mask = _mask_arg(key_padding_mask, B, S_k, dev)
    if alibi_slopes is not None:
        _need(alibi_slopes, "alibi_slopes", torch.float32, (H_q,), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H_q, 1), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H_q, 1), dev)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    return dev, (B, S_k, H_q, H_kv, D), mask, out, lse, sc


def attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                scale: Optional[float] = None, key_padding_mask: Optional[torch.Tensor] = None,
                alibi_slopes: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                return_lse: bool = True):
    """Single-token attention through ``sa_attn_decode`` (split-KV + merge).

    q ``[B, 1, H_q, D]``; k_cache/v_cache ``[B, S_k, H_kv, D]``.  Returns
    ``out [B, 1, H_q, D]`` (and float32 ``lse [B, H_q, 1]``).
    """
    dev, (B, S_k, H_q, H_kv, D), mask, out, lse, sc = _decode_prepare(
        q, k_cache, v_cache, key_padding_mask, alibi_slopes, out, lse, return_lse, scale)
    if workspace is None:
        workspace = decode_workspace(B, H_q, S_k, D, dev)
    _need(workspace, "workspace", None, None, dev)
    st = lib().sa_attn_decode(q.data_ptr(), _ptr(k_cache), _ptr(v_cache), out.data_ptr(), _ptr(lse),
                              B, S_k, H_q, H_kv, D, sc, _ptr(mask), _ptr(alibi_slopes),
                              _DTYPE[q.dtype], workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st)
    return (out, lse) if return_lse else out


def attn_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                        scale: Optional[float] = None, key_padding_mask: Optional[torch.Tensor] = None,
                        alibi_slopes: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, return_lse: bool = True):
    """``attn_decode`` through ``sa_attn_decode_noalloc``: the library keeps
    the partial results in its own scratch, so no workspace is passed and the
    C call allocates nothing (pass ``out`` and ``lse`` to allocate nothing
    here either).  Calls that may overlap on one GPU must not be issued."""
    dev, (B, S_k, H_q, H_kv, D), mask, out, lse, sc = _decode_prepare(
        q, k_cache, v_cache, key_padding_mask, alibi_slopes, out, lse, return_lse, scale)
    st = lib().sa_attn_decode_noalloc(q.data_ptr(), _ptr(k_cache), _ptr(v_cache), out.data_ptr(), _ptr(lse),
                                      B, S_k, H_q, H_kv, D, sc, _ptr(mask), _ptr(alibi_slopes),
                                      _DTYPE[q.dtype], _stream(dev))
    _check(st)
    return (out, lse) if return_lse else out


def decode_fused_workspace(B: int, H_q: int, S_k: int, D: int, device) -> torch.Tensor:
    """A zeroed device byte buffer for ``attn_decode_fused`` at these sizes
    (its arrival counters must start at zero; calls leave them zero again)."""
    n = int(lib().sa_attn_decode_fused_workspace_size(B, H_q, S_k, D))
    return torch.zeros(max(n, DECODE_ARRIVE_BYTES), dtype=torch.uint8, device=device)


def attn_decode_fused(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      scale: Optional[float] = None, key_padding_mask: Optional[torch.Tensor] = None,
                      alibi_slopes: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                      return_lse: bool = True):
    """Single-token attention through ``sa_attn_decode_fused`` (one kernel:
    the last split of each head group to finish merges it).  As
    ``attn_decode``; a ``workspace``
    passed in must come from ``decode_fused_workspace`` (or be zeroed the same
    way) and be reused only by calls ordered on one stream."""
    dev, (B, S_k, H_q, H_kv, D), mask, out, lse, sc = _decode_prepare(
        q, k_cache, v_cache, key_padding_mask, alibi_slopes, out, lse, return_lse, scale)
    if workspace is None:
        workspace = decode_fused_workspace(B, H_q, S_k, D, dev)
    _need(workspace, "workspace", None, None, dev)
    st = lib().sa_attn_decode_fused(q.data_ptr(), _ptr(k_cache), _ptr(v_cache), out.data_ptr(), _ptr(lse),
                                    B, S_k, H_q, H_kv, D, sc, _ptr(mask), _ptr(alibi_slopes),
                                    _DTYPE[q.dtype], workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(dev))
    _check(st)
    return (out, lse) if return_lse else out


def bwd_workspace_size(B: int, H_q: int, S_q: int) -> int:
    return int(lib().sa_attn_bwd_workspace_size(B, H_q, S_q))


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
             dout: torch.Tensor, lse: torch.Tensor, causal: bool = False,
             scale: Optional[float] = None, key_padding_mask: Optional[torch.Tensor] = None,
             alibi_slopes: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None):
    """Gradients of ``attn_fwd``'s output through ``sa_attn_bwd``.

    ``out`` and ``lse`` are what ``attn_fwd`` returned for the same inputs;
    ``dout`` has the shape of ``out``.  Returns ``(dq, dk, dv)``.
    """
    _need(q, "q")
    if q.dtype not in _DTYPE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    dev = q.device
    B, S_q, H_q, D = q.shape
    _need(k, "k", q.dtype, None, dev)
    if k.dim() != 4 or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k has shape {tuple(k.shape)}, incompatible with q {tuple(q.shape)}")
    S_k, H_kv = k.shape[1], k.shape[2]
    _need(v, "v", q.dtype, k.shape, dev)
    _need(out, "out", q.dtype, q.shape, dev)
    _need(dout, "dout", q.dtype, q.shape, dev)
    _need(lse, "lse", torch.float32, (B, H_q, S_q), dev)
    mask = _mask_arg(key_padding_mask, B, S_k, dev)
    if alibi_slopes is not None:
        _need(alibi_slopes, "alibi_slopes", torch.float32, (H_q,), dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", q.dtype, q.shape, dev)
    _need(dk, "dk", q.dtype, k.shape, dev)
    _need(dv, "dv", q.dtype, k.shape, dev)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_size(B, H_q, S_q), 16), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", None, None, dev)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    st = lib().sa_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                           _ptr(dq), _ptr(dk), _ptr(dv), B, S_q, S_k, H_q, H_kv, D, sc,
                           int(bool(causal)), _ptr(mask), _ptr(alibi_slopes), _DTYPE[q.dtype],
                           workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                           _stream(dev))
    _check(st)
    return dq, dk, dv


__all__ = ["attn_fwd", "attn_fwd_block_sparse", "attn_fwd_ext", "SPARSE_BLOCK", "attn_decode",
           "attn_decode_fused", "decode_fused_workspace", "attn_bwd", "bwd_workspace_size", "decode_workspace_size", "decode_num_splits",
           "decode_workspace", "lib", "last_error", "status_string", "SaAttnError",
           "SIGNATURES", "LIB_PATH", "SA_OK", "SA_ERR_INVALID_ARG", "SA_ERR_UNSUPPORTED",
           "SA_ERR_WORKSPACE", "SA_ERR_HIP", "SA_F16", "SA_BF16"]
