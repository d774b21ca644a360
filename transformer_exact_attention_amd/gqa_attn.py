"""Python binding of libgqa_attn (ctypes).

Argument marshalling only: every step of attention runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  The functions
carry the C names; tensors in, status codes turned into exceptions.

The library is loaded from this package's directory.  If it is missing the
first call raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch  # noqa: F401  (loads the HIP runtime the library shares)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa_attn.so")

GQA_OK, GQA_ERR_INVALID_ARG, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP, GQA_ERR_OUT_OF_BLOCKS = range(6)
GQA_F32, GQA_BF16 = 0, 1
PAGE_BLOCK_SIZE = 16

EXPORTS = ("gqa_attn_abi_version", "gqa_attn_status_string", "attn_prefill_fwd",
           "attn_decode_workspace_bytes", "attn_decode_fwd", "attn_decode_validate",
           "gqa_kv_pool_create", "gqa_kv_pool_destroy", "gqa_kv_pool_free_blocks", "gqa_kv_seq_new",
           "gqa_kv_seq_fork", "gqa_kv_seq_release", "gqa_kv_seq_len", "gqa_kv_reserve", "gqa_kv_block_table",
           "attn_kv_append", "attn_kv_copy_blocks", "attn_decode_fp8_fwd", "attn_kv_append_fp8",
           "attn_kv_copy_blocks_fp8", "attn_prefill_window_fwd", "attn_decode_window_fwd",
           "attn_prefill_lse_fwd", "attn_prefill_bwd_workspace_bytes", "attn_prefill_bwd",
           "attn_decode_fwd_noalloc")

DECODE_NOALLOC_MAX_BYTES = 64 << 20      # GQA_DECODE_NOALLOC_MAX_BYTES

_lib = None


class GqaAttnError(RuntimeError):
    pass


class OutOfBlocksError(GqaAttnError):
    """A KV pool has too few free blocks (or sequence ids) for the request."""


def load_library(path: str = LIB_PATH):
    """Load (once) and type the C entry points.  Raises if the library is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libgqa_attn not built: {path} is missing "
                          "(run `python -m transformer_exact_attention_amd.build`)")
    lib = ctypes.CDLL(path)
    c_int, c_float, c_size, vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    lib.gqa_attn_abi_version.restype = c_int
    lib.gqa_attn_abi_version.argtypes = []
    lib.gqa_attn_status_string.restype = ctypes.c_char_p
    lib.gqa_attn_status_string.argtypes = [c_int]
    lib.attn_prefill_fwd.restype = c_int
    lib.attn_prefill_fwd.argtypes = [vp, vp, vp, vp] + [c_int] * 6 + [c_float, c_int, c_int, vp]
    lib.attn_decode_workspace_bytes.restype = c_size
    lib.attn_decode_workspace_bytes.argtypes = [c_int] * 4
    lib.attn_decode_fwd.restype = c_int
    lib.attn_decode_fwd.argtypes = [vp, vp, vp, vp, vp, vp] + [c_int] * 7 + [c_float, c_int, vp, c_size, vp]
    lib.attn_decode_fwd_noalloc.restype = c_int
    lib.attn_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp] + [c_int] * 7 + [c_float, c_int, vp]
    lib.attn_decode_validate.restype = c_int
    lib.attn_decode_validate.argtypes = [vp, vp] + [c_int] * 5 + [vp]
    ip = ctypes.POINTER(c_int)
    lib.gqa_kv_pool_create.restype = c_int
    lib.gqa_kv_pool_create.argtypes = [c_int, c_int, c_int, ctypes.POINTER(vp)]
    lib.gqa_kv_pool_destroy.restype = None
    lib.gqa_kv_pool_destroy.argtypes = [vp]
    lib.gqa_kv_pool_free_blocks.restype = c_int
    lib.gqa_kv_pool_free_blocks.argtypes = [vp]
    lib.gqa_kv_seq_new.restype = c_int
    lib.gqa_kv_seq_new.argtypes = [vp, ip]
    lib.gqa_kv_seq_fork.restype = c_int
    lib.gqa_kv_seq_fork.argtypes = [vp, c_int, ip]
    lib.gqa_kv_seq_release.restype = c_int
    lib.gqa_kv_seq_release.argtypes = [vp, c_int]
    lib.gqa_kv_seq_len.restype = c_int
    lib.gqa_kv_seq_len.argtypes = [vp, c_int]
    lib.gqa_kv_reserve.restype = c_int
    lib.gqa_kv_reserve.argtypes = [vp, vp, vp, c_int, vp, vp, vp, ip]
    lib.gqa_kv_block_table.restype = c_int
    lib.gqa_kv_block_table.argtypes = [vp, vp, c_int, vp, c_int, vp]
    lib.attn_kv_append.restype = c_int
    lib.attn_kv_append.argtypes = [vp, vp, vp, vp, vp] + [c_int] * 5 + [vp]
    lib.attn_kv_copy_blocks.restype = c_int
    lib.attn_kv_copy_blocks.argtypes = [vp, vp, vp, vp] + [c_int] * 5 + [vp]
    lib.attn_prefill_window_fwd.restype = c_int
    lib.attn_prefill_window_fwd.argtypes = [vp, vp, vp, vp] + [c_int] * 6 + [c_float, c_int, c_int, vp]
    lib.attn_decode_window_fwd.restype = c_int
    lib.attn_decode_window_fwd.argtypes = [vp, vp, vp, vp, vp, vp] + [c_int] * 7 + [c_float, c_int, c_int, vp,
                                                                                   c_size, vp]
    lib.attn_decode_fp8_fwd.restype = c_int
    lib.attn_decode_fp8_fwd.argtypes = [vp] * 8 + [c_int] * 7 + [c_float, vp, c_size, vp]
    lib.attn_kv_append_fp8.restype = c_int
    lib.attn_kv_append_fp8.argtypes = [vp] * 7 + [c_int] * 4 + [vp]
    lib.attn_kv_copy_blocks_fp8.restype = c_int
    lib.attn_kv_copy_blocks_fp8.argtypes = [vp] * 6 + [c_int] * 4 + [vp]
    lib.attn_prefill_lse_fwd.restype = c_int
    lib.attn_prefill_lse_fwd.argtypes = [vp] * 5 + [c_int] * 6 + [c_float, c_int, c_int, c_int, vp]
    lib.attn_prefill_bwd_workspace_bytes.restype = c_size
    lib.attn_prefill_bwd_workspace_bytes.argtypes = [c_int] * 3
    lib.attn_prefill_bwd.restype = c_int
    lib.attn_prefill_bwd.argtypes = [vp] * 9 + [c_int] * 6 + [c_float, c_int, c_int, c_int, vp, c_size, vp]
    _lib = lib
    return lib


def gqa_attn_abi_version() -> int:
    return load_library().gqa_attn_abi_version()


def gqa_attn_status_string(status: int) -> str:
    return load_library().gqa_attn_status_string(int(status)).decode()


def _raise(status: int, what: str):
    if status == GQA_OK:
        return
    msg = f"{what}: {gqa_attn_status_string(status)} (status {status})"
    if status == GQA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if status == GQA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status == GQA_ERR_OUT_OF_BLOCKS:
        raise OutOfBlocksError(msg)
    raise GqaAttnError(msg)


_DTYPES = {torch.float32: GQA_F32, torch.bfloat16: GQA_BF16}


def _dtype_code(*ts) -> int:
    dt = ts[0].dtype
    if any(t.dtype != dt for t in ts):
        raise ValueError("q/k/v/o must share one dtype")
    if dt not in _DTYPES:
        raise NotImplementedError(f"dtype {dt} not supported (float32, bfloat16)")
    return _DTYPES[dt]


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def attn_prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: Optional[torch.Tensor] = None, *,
                     scale: Optional[float] = None, causal: bool = False, stream=None,
                     window: Optional[int] = None) -> torch.Tensor:
    """O = softmax(Q K^T * scale) V with grouped K/V heads; q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d].

    ``scale`` defaults to 1/sqrt(d).  ``window`` (>= 1): causal sliding
    window, each query sees its last ``window`` keys (attn_prefill_window_fwd).
    Returns ``o`` (allocated when None).
    """
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, d]")
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k and v")
    if o is None:
        o = torch.empty_like(q)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    _dev(q, k, v, o)
    code = _dtype_code(q, k, v, o)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if window is not None:
        st = lib.attn_prefill_window_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, Hq, Hkv, Sq, Sk,
                                         d, float(scale), int(window), code, _stream(stream))
        _raise(st, "attn_prefill_window_fwd")
        return o
    st = lib.attn_prefill_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, Hq, Hkv, Sq, Sk, d,
                              float(scale), 1 if causal else 0, code, _stream(stream))
    _raise(st, "attn_prefill_fwd")
    return o


def attn_prefill_window_fwd(q, k, v, o=None, *, window: int, scale=None, stream=None):
    """Causal sliding-window attention: each query sees its last ``window`` keys."""
    return attn_prefill_fwd(q, k, v, o, scale=scale, causal=True, stream=stream, window=window)


def _prefill_shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, d]")
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k and v")
    return B, Hq, Hkv, Sq, Sk, d


def attn_prefill_lse_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None, *, scale: Optional[float] = None, causal: bool = False,
                         window: int = 0, stream=None):
    """Forward that also returns the per-row natural-log log-sum-exp [B, Hq, Sq] (fp32).

    Same output as attn_prefill_fwd (window 0) or attn_prefill_window_fwd
    (window >= 1, causal implied).  Returns ``(o, lse)``.
    """
    lib = load_library()
    B, Hq, Hkv, Sq, Sk, d = _prefill_shapes(q, k, v)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if tuple(o.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32:
        raise ValueError("o must have q's shape and lse be float32 [B, Hq, Sq]")
    _dev(q, k, v, o, lse)
    code = _dtype_code(q, k, v, o)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.attn_prefill_lse_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
                                  Sq, Sk, d, float(scale), 1 if causal else 0, int(window), code, _stream(stream))
    _raise(st, "attn_prefill_lse_fwd")
    return o, lse


def attn_prefill_bwd_workspace_bytes(B: int, Hq: int, Sq: int) -> int:
    return int(load_library().attn_prefill_bwd_workspace_bytes(B, Hq, Sq))


def attn_prefill_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                     dout: torch.Tensor, dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                     dv: Optional[torch.Tensor] = None, *, scale: Optional[float] = None, causal: bool = False,
                     window: int = 0, workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients (dq, dk, dv) of attn_prefill_lse_fwd for output gradient ``dout`` (bf16).

    ``o`` and ``lse`` are the forward's outputs for the same q, k, v, scale,
    causal and window.  Returns ``(dq, dk, dv)`` (allocated when None).
    """
    lib = load_library()
    B, Hq, Hkv, Sq, Sk, d = _prefill_shapes(q, k, v)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape) or tuple(dq.shape) != tuple(q.shape):
        raise ValueError("o, dout and dq must have q's shape")
    if tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(k.shape):
        raise ValueError("dk and dv must have k's shape")
    if tuple(lse.shape) != (B, Hq, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, Sq]")
    _dev(q, k, v, o, lse, dout, dq, dk, dv)
    code = _dtype_code(q, k, v, o, dout, dq, dk, dv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_prefill_bwd_workspace_bytes(B, Hq, Sq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _dev(workspace)
    st = lib.attn_prefill_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Sq, Sk, d,
                              float(scale), 1 if causal else 0, int(window), code, workspace.data_ptr(),
                              workspace.numel() * workspace.element_size(), _stream(stream))
    _raise(st, "attn_prefill_bwd")
    return dq, dk, dv


def attn_decode_workspace_bytes(B: int, Hq: int, d: int, max_seq_len: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, Hq, d, max_seq_len))


def decode_workspace(B: int, Hq: int, d: int, max_seq_len: int, device="cuda") -> torch.Tensor:
    """A byte tensor large enough for attn_decode_fwd (torch allocations are 256-byte aligned)."""
    return torch.empty(attn_decode_workspace_bytes(B, Hq, d, max_seq_len), dtype=torch.uint8, device=device)


def attn_decode_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                    o: Optional[torch.Tensor] = None, *, block_table: Optional[torch.Tensor] = None,
                    max_seq_len: Optional[int] = None, scale: Optional[float] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None,
                    window: Optional[int] = None) -> torch.Tensor:
    """One query token per sequence over a contiguous or paged KV cache
    (``window``: only each sequence's last ``window`` tokens, attn_decode_window_fwd).

    q [B,Hq,d]; contiguous k/v_cache [B,Hkv,S_max,d]; paged k/v_cache
    [num_blocks,Hkv,16,d] with block_table int32 [B,max_blocks].  seq_lens
    int32 [B] on the device.  ``max_seq_len`` defaults to S_max (contiguous) or
    16*max_blocks (paged).
    """
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q must be [B,Hq,d]; k_cache and v_cache 4-D and equal in shape")
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[3] != d:
        raise ValueError("head dim mismatch")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    tensors = [q, k_cache, v_cache, seq_lens]
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B, max_blocks]")
        if k_cache.shape[2] != PAGE_BLOCK_SIZE:
            raise ValueError("paged caches hold 16 tokens per block")
        max_blocks = block_table.shape[1]
        if max_seq_len is None:
            max_seq_len = max_blocks * PAGE_BLOCK_SIZE
        tensors.append(block_table)
        bt_ptr = block_table.data_ptr()
        block_size = PAGE_BLOCK_SIZE
    else:
        if k_cache.shape[0] != B:
            raise ValueError("contiguous cache must be [B,Hkv,S_max,d]")
        max_blocks = 0
        block_size = 0
        if max_seq_len is None:
            max_seq_len = k_cache.shape[2]
        if max_seq_len != k_cache.shape[2]:
            raise ValueError("contiguous cache: max_seq_len must equal S_max")
        bt_ptr = None
    if o is None:
        o = torch.empty_like(q)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    tensors.append(o)
    _dev(*tensors)
    code = _dtype_code(q, k_cache, v_cache, o)
    if workspace is None:
        workspace = decode_workspace(B, Hq, d, max_seq_len, q.device)
    _dev(workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if window is not None:
        st = lib.attn_decode_window_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
                                        seq_lens.data_ptr(), bt_ptr, B, Hq, Hkv, d, int(max_seq_len), block_size,
                                        max_blocks, float(scale), int(window), code, workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream(stream))
        _raise(st, "attn_decode_window_fwd")
        return o
    st = lib.attn_decode_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
                             seq_lens.data_ptr(), bt_ptr, B, Hq, Hkv, d, int(max_seq_len), block_size,
                             max_blocks, float(scale), code, workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), _stream(stream))
    _raise(st, "attn_decode_fwd")
    return o


def attn_decode_fwd_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                            o: torch.Tensor, *, block_table: Optional[torch.Tensor] = None,
                            max_seq_len: Optional[int] = None, scale: Optional[float] = None,
                            stream=None) -> torch.Tensor:
    """attn_decode_fwd without a workspace: the library keeps the partial results
    in its static device scratch (nothing is allocated, here or in the library).

    The caller passes the output ``o``.  Sizes whose workspace would exceed
    DECODE_NOALLOC_MAX_BYTES raise GqaAttnError.  Calls that overlap on one GPU
    share the scratch and race.
    """
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q must be [B,Hq,d]; k_cache and v_cache 4-D and equal in shape")
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[3] != d or tuple(o.shape) != tuple(q.shape):
        raise ValueError("head dim mismatch, or o not of q's shape")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    tensors = [q, k_cache, v_cache, seq_lens, o]
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B, max_blocks]")
        max_blocks, block_size = block_table.shape[1], PAGE_BLOCK_SIZE
        max_seq_len = max_blocks * PAGE_BLOCK_SIZE if max_seq_len is None else max_seq_len
        tensors.append(block_table)
        bt_ptr = block_table.data_ptr()
    else:
        max_blocks, block_size = 0, 0
        max_seq_len = k_cache.shape[2] if max_seq_len is None else max_seq_len
        if max_seq_len != k_cache.shape[2] or k_cache.shape[0] != B:
            raise ValueError("contiguous cache must be [B,Hkv,S_max,d] with max_seq_len == S_max")
        bt_ptr = None
    _dev(*tensors)
    code = _dtype_code(q, k_cache, v_cache, o)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.attn_decode_fwd_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
                                     seq_lens.data_ptr(), bt_ptr, B, Hq, Hkv, d, int(max_seq_len), block_size,
                                     max_blocks, float(scale), code, _stream(stream))
    _raise(st, "attn_decode_fwd_noalloc")
    return o


def attn_decode_window_fwd(q, k_cache, v_cache, seq_lens, o=None, *, window: int, **kw):
    """Decode attending only each sequence's last ``window`` cached tokens."""
    return attn_decode_fwd(q, k_cache, v_cache, seq_lens, o, window=window, **kw)


def attn_decode_validate(seq_lens: torch.Tensor, block_table: Optional[torch.Tensor], max_seq_len: int,
                         num_physical_blocks: int = 0, stream=None) -> int:
    """Synchronous check of device lengths / table entries; returns the status code."""
    lib = load_library()
    B = seq_lens.shape[0]
    mb = block_table.shape[1] if block_table is not None else 0
    bs = PAGE_BLOCK_SIZE if block_table is not None else 0
    return lib.attn_decode_validate(seq_lens.data_ptr(), block_table.data_ptr() if block_table is not None else None,
                                    B, int(max_seq_len), bs, mb, int(num_physical_blocks), _stream(stream))


# ---- paged KV cache (gqa_kv_cache.h) ---------------------------------------

def _host_i32(a, n=None):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    if n is not None and a.shape != (n,):
        raise ValueError(f"expected {n} int32 values")
    return a


class KVPool:
    """Host-side page allocator of the library (gqa_kv_pool): page tables,
    block references, copy-on-write prefix sharing.  Methods carry the C
    names without the ``gqa_kv_`` prefix; ids and slots are plain ints and
    int32 numpy arrays."""

    def __init__(self, num_blocks: int, max_seqs: int, max_blocks_per_seq: int):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _raise(self._lib.gqa_kv_pool_create(int(num_blocks), int(max_seqs), int(max_blocks_per_seq),
                                            ctypes.byref(h)), "gqa_kv_pool_create")
        self._h = h
        self.num_blocks, self.max_seqs, self.max_blocks_per_seq = int(num_blocks), int(max_seqs), int(max_blocks_per_seq)

    def close(self):
        if getattr(self, "_h", None):
            self._lib.gqa_kv_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def free_blocks(self) -> int:
        return int(self._lib.gqa_kv_pool_free_blocks(self._h))

    def seq_new(self) -> int:
        out = ctypes.c_int()
        _raise(self._lib.gqa_kv_seq_new(self._h, ctypes.byref(out)), "gqa_kv_seq_new")
        return out.value

    def seq_fork(self, parent: int) -> int:
        out = ctypes.c_int()
        _raise(self._lib.gqa_kv_seq_fork(self._h, int(parent), ctypes.byref(out)), "gqa_kv_seq_fork")
        return out.value

    def seq_release(self, seq: int):
        _raise(self._lib.gqa_kv_seq_release(self._h, int(seq)), "gqa_kv_seq_release")

    def seq_len(self, seq: int) -> int:
        return int(self._lib.gqa_kv_seq_len(self._h, int(seq)))

    def reserve(self, seqs, counts):
        """Slots for counts[i] new tokens of seqs[i]; returns (slots, copy_src, copy_dst)."""
        import numpy as np
        seqs = _host_i32(seqs)
        counts = _host_i32(counts, seqs.shape[0])
        n = seqs.shape[0]
        total = int(counts.sum()) if n else 0
        slots = np.empty(max(total, 1), dtype=np.int32)
        src = np.empty(max(n, 1), dtype=np.int32)
        dst = np.empty(max(n, 1), dtype=np.int32)
        nc = ctypes.c_int(0)
        _raise(self._lib.gqa_kv_reserve(self._h, seqs.ctypes.data, counts.ctypes.data, n, slots.ctypes.data,
                                        src.ctypes.data, dst.ctypes.data, ctypes.byref(nc)), "gqa_kv_reserve")
        return slots[:total].copy(), src[:nc.value].copy(), dst[:nc.value].copy()

    def block_table(self, seqs, max_blocks: int):
        """(table int32 [n, max_blocks] padded with -1, lens int32 [n])."""
        import numpy as np
        seqs = _host_i32(seqs)
        n = seqs.shape[0]
        table = np.empty((n, int(max_blocks)), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        _raise(self._lib.gqa_kv_block_table(self._h, seqs.ctypes.data, n, table.ctypes.data, int(max_blocks),
                                            lens.ctypes.data), "gqa_kv_block_table")
        return table, lens


def _page_dims(k_cache, v_cache):
    if k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[2] != PAGE_BLOCK_SIZE:
        raise ValueError("k_cache and v_cache must both be [num_blocks, Hkv, 16, d]")
    num_blocks, Hkv, _, d = k_cache.shape
    return num_blocks, Hkv, d


def attn_kv_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   slots: torch.Tensor, stream=None):
    """Write tokens k_new/v_new [n, Hkv, d] into the pages at slots (int32 [n], device)."""
    lib = load_library()
    num_blocks, Hkv, d = _page_dims(k_cache, v_cache)
    n = k_new.shape[0]
    if k_new.dim() != 3 or tuple(k_new.shape) != (n, Hkv, d) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new and v_new must both be [n_tokens, Hkv, d]")
    if slots.dtype != torch.int32 or tuple(slots.shape) != (n,):
        raise ValueError("slots must be int32 [n_tokens]")
    if n == 0:
        return
    _dev(k_cache, v_cache, k_new, v_new, slots)
    code = _dtype_code(k_cache, v_cache, k_new, v_new)
    _raise(lib.attn_kv_append(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                              slots.data_ptr(), n, num_blocks, Hkv, d, code, _stream(stream)), "attn_kv_append")


def attn_kv_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, src: torch.Tensor, dst: torch.Tensor,
                        stream=None):
    """Copy whole blocks src[i] -> dst[i] (int32 [n], device) of both caches."""
    lib = load_library()
    num_blocks, Hkv, d = _page_dims(k_cache, v_cache)
    n = src.shape[0]
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.dim() != 1 or tuple(dst.shape) != (n,):
        raise ValueError("src and dst must be int32 [n]")
    if n == 0:
        return
    _dev(k_cache, v_cache, src, dst)
    code = _dtype_code(k_cache, v_cache)
    _raise(lib.attn_kv_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), src.data_ptr(), dst.data_ptr(), n,
                                   num_blocks, Hkv, d, code, _stream(stream)), "attn_kv_copy_blocks")


# ---- fp8 KV caches (E4M3 codes + one fp32 scale per row) -------------------

def _fp8_pages(k_cache, v_cache, k_scale, v_scale):
    num_blocks, Hkv, d = _page_dims(k_cache, v_cache)
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("fp8 caches hold uint8 E4M3 codes")
    for sc in (k_scale, v_scale):
        if sc.dtype != torch.float32 or tuple(sc.shape) != (num_blocks, Hkv, PAGE_BLOCK_SIZE):
            raise ValueError("fp8 scales must be float32 [num_blocks, Hkv, 16]")
    return num_blocks, Hkv, d


def attn_kv_append_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                       k_new: torch.Tensor, v_new: torch.Tensor, slots: torch.Tensor, stream=None):
    """Quantise bf16 tokens [n, Hkv, d] into fp8 pages and their row scales at slots."""
    lib = load_library()
    num_blocks, Hkv, d = _fp8_pages(k_cache, v_cache, k_scale, v_scale)
    n = k_new.shape[0]
    if k_new.dim() != 3 or tuple(k_new.shape) != (n, Hkv, d) or tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new and v_new must both be [n_tokens, Hkv, d]")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise ValueError("new tokens are bfloat16")
    if slots.dtype != torch.int32 or tuple(slots.shape) != (n,):
        raise ValueError("slots must be int32 [n_tokens]")
    if n == 0:
        return
    _dev(k_cache, v_cache, k_scale, v_scale, k_new, v_new, slots)
    _raise(lib.attn_kv_append_fp8(k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(),
                                  k_new.data_ptr(), v_new.data_ptr(), slots.data_ptr(), n, num_blocks, Hkv, d,
                                  _stream(stream)), "attn_kv_append_fp8")


def attn_kv_copy_blocks_fp8(k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                            v_scale: torch.Tensor, src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Copy whole fp8 blocks src[i] -> dst[i] with their row scales."""
    lib = load_library()
    num_blocks, Hkv, d = _fp8_pages(k_cache, v_cache, k_scale, v_scale)
    n = src.shape[0]
    if src.dtype != torch.int32 or dst.dtype != torch.int32 or src.dim() != 1 or tuple(dst.shape) != (n,):
        raise ValueError("src and dst must be int32 [n]")
    if n == 0:
        return
    _dev(k_cache, v_cache, k_scale, v_scale, src, dst)
    _raise(lib.attn_kv_copy_blocks_fp8(k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(),
                                       v_scale.data_ptr(), src.data_ptr(), dst.data_ptr(), n, num_blocks, Hkv, d,
                                       _stream(stream)), "attn_kv_copy_blocks_fp8")


def attn_decode_fp8_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: torch.Tensor,
                        v_scale: torch.Tensor, seq_lens: torch.Tensor, o: Optional[torch.Tensor] = None, *,
                        block_table: Optional[torch.Tensor] = None, max_seq_len: Optional[int] = None,
                        scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """attn_decode_fwd over an fp8 cache: uint8 codes laid out like the bf16
    caches, fp32 scales [B,Hkv,S_max] (contiguous) or [num_blocks,Hkv,16]
    (paged); q and o bf16."""
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4 or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q must be [B,Hq,d]; k_cache and v_cache 4-D and equal in shape")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("fp8 caches hold uint8 E4M3 codes")
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[3] != d:
        raise ValueError("head dim mismatch")
    if tuple(k_scale.shape) != tuple(k_cache.shape[:3]) or tuple(v_scale.shape) != tuple(k_scale.shape):
        raise ValueError("scales must have the cache's shape without d")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32:
        raise ValueError("scales are float32")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    tensors = [q, k_cache, v_cache, k_scale, v_scale, seq_lens]
    if block_table is not None:
        if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be int32 [B, max_blocks]")
        if k_cache.shape[2] != PAGE_BLOCK_SIZE:
            raise ValueError("paged caches hold 16 tokens per block")
        max_blocks = block_table.shape[1]
        if max_seq_len is None:
            max_seq_len = max_blocks * PAGE_BLOCK_SIZE
        tensors.append(block_table)
        bt_ptr = block_table.data_ptr()
        block_size = PAGE_BLOCK_SIZE
    else:
        if k_cache.shape[0] != B:
            raise ValueError("contiguous cache must be [B,Hkv,S_max,d]")
        max_blocks = 0
        block_size = 0
        if max_seq_len is None:
            max_seq_len = k_cache.shape[2]
        if max_seq_len != k_cache.shape[2]:
            raise ValueError("contiguous cache: max_seq_len must equal S_max")
        bt_ptr = None
    if q.dtype != torch.bfloat16:
        raise ValueError("q is bfloat16")
    if o is None:
        o = torch.empty_like(q)
    if tuple(o.shape) != tuple(q.shape) or o.dtype != torch.bfloat16:
        raise ValueError("o must be bfloat16 with q's shape")
    tensors.append(o)
    _dev(*tensors)
    if workspace is None:
        workspace = decode_workspace(B, Hq, d, max_seq_len, q.device)
    _dev(workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.attn_decode_fp8_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(),
                                 v_scale.data_ptr(), o.data_ptr(), seq_lens.data_ptr(), bt_ptr, B, Hq, Hkv, d,
                                 int(max_seq_len), block_size, max_blocks, float(scale), workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), _stream(stream))
    _raise(st, "attn_decode_fp8_fwd")
    return o
