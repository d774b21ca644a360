"""Seeded synthetic inputs for the attention path.

This module is shared by the tests, the benchmark and ``smoke()``.  It holds no
attention arithmetic: it only draws iid N(0,1) values (the pages' demo feeds
``randn`` tensors to attention, [Attention variants deep-dive, §5 GQA code]),
rounds them to bfloat16 bit patterns, draws per-sequence cache lengths and a
random physical placement of 16-token KV blocks behind a per-sequence block
table ([Different attention mechanisms, §5 Page Attention, steps 1-2]).

Seeds: workload ``k`` draws stream ``s`` from ``numpy.random.default_rng([k, s])``
(values: chunk ``i`` of 2^22 elements from ``default_rng([k, s, i])``) with
s = 0 (q), 1 (k), 2 (v), 3 (lengths), 4 (block permutation).

Everything is returned as numpy arrays: float32 for fp32 workloads, uint16
bfloat16 bit patterns for bf16 workloads, int32 for lengths and tables.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BLOCK_SIZE = 16          # tokens per KV page
STREAM_Q, STREAM_K, STREAM_V, STREAM_LENS, STREAM_PERM = 0, 1, 2, 3, 4
_CHUNK = 1 << 22
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


# ----------------------------------------------------------------------------
# bfloat16 encoding of the drawn values (input generation, not attention math)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the uint16 bit patterns.  NaN maps to the quiet NaN 0x7FC0 (with
    its sign); overflow past the largest finite bfloat16 becomes +-inf, as the
    rounding rule requires.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    with np.errstate(over="ignore"):
        r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)).astype(np.uint16) & np.uint16(0x8000)) | np.uint16(0x7FC0)
    return r


def _fill_chunks(seed, n: int, out: np.ndarray, convert) -> None:
    """Fill ``out`` (length n) chunk by chunk; chunk i draws from default_rng([*seed, i]).

    Chunks are independent streams, so they are drawn on a few threads (numpy
    releases the GIL while it fills an array).  The values depend only on the
    seed and the fixed chunk size, never on the thread count.
    """
    seed = list(seed) if isinstance(seed, (list, tuple)) else [int(seed)]
    starts = list(range(0, n, _CHUNK))

    def one(i):
        s = starts[i]
        e = min(n, s + _CHUNK)
        out[s:e] = convert(np.random.default_rng(seed + [i]).standard_normal(e - s, dtype=np.float32))

    if len(starts) <= 1:
        for i in range(len(starts)):
            one(i)
        return
    with ThreadPoolExecutor(max_workers=min(_THREADS, len(starts))) as ex:
        list(ex.map(one, range(len(starts))))


def normal_f32(seed, shape) -> np.ndarray:
    """iid N(0,1) float32 values of ``shape`` (seed: int or list of ints)."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, np.float32)
    _fill_chunks(seed, n, out, lambda x: x)
    return out.reshape(shape)


def normal_bf16(seed, shape) -> np.ndarray:
    """The same draws as :func:`normal_f32`, rounded to bfloat16; uint16 bit patterns."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, np.uint16)
    _fill_chunks(seed, n, out, f32_to_bf16_bits)
    return out.reshape(shape)


def normal(seed, shape, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return normal_f32(seed, shape)
    if dtype == "bf16":
        return normal_bf16(seed, shape)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    dtype: str
    causal: bool
    scale: Optional[float] = None

    @property
    def scale_value(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """4*d*Hq*B per unmasked (query, key) pair: QK^T and PV, 2 FLOP per MAC."""
        if self.causal:
            off = self.Sk - self.Sq
            pairs = sum(min(self.Sk, i + off + 1) for i in range(self.Sq))
        else:
            pairs = self.Sq * self.Sk
        return 4.0 * self.d * self.Hq * self.B * pairs

    def io_bytes(self) -> int:
        e = 4 if self.dtype == "f32" else 2
        return e * self.d * (2 * self.B * self.Hq * self.Sq + 2 * self.B * self.Hkv * self.Sk)


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    d: int
    L_lo: int
    L_hi: int
    paged: bool
    S_max: int = 0               # contiguous cache length (>= L_hi)
    dtype: str = "bf16"
    scale: Optional[float] = None

    @property
    def scale_value(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    @property
    def max_blocks(self) -> int:
        return -(-self.L_hi // BLOCK_SIZE)


CFG1 = PrefillWorkload("gqa_tiny_f32_B1_Hq4_Hkv2_S128_d64", 1, 1, 4, 2, 128, 128, 64, "f32", False)
CFG2 = PrefillWorkload("mha_causal_prefill_B4_H32_S2048_d128", 2, 4, 32, 32, 2048, 2048, 128, "bf16", True)
CFG3 = PrefillWorkload("gqa_causal_prefill_B2_Hq32_Hkv8_S8192_d128", 3, 2, 32, 8, 8192, 8192, 128, "bf16", True)
CFG4 = DecodeWorkload("gqa_decode_contig_B64_Hq32_Hkv8_d128_L512-4096", 4, 64, 32, 8, 128, 512, 4096, False, S_max=4096)


def cfg5(Hkv: int) -> DecodeWorkload:
    return DecodeWorkload(f"paged_decode_B16_Hq32_Hkv{Hkv}_d128_L8192-32768", 5, 16, 32, Hkv, 128,
                          8192, 32768, True)


# Long context: LLaMA-3-8B-shaped attention (32 query heads, 8 K/V heads,
# d 128) at 32K positions [Attention variants deep-dive, §8 Q4]; a sweep
# point beside the prefill workloads, not a parity configuration.
LONG_CONTEXT = PrefillWorkload("gqa_causal_prefill_B1_Hq32_Hkv8_S32768_d128", 6, 1, 32, 8, 32768, 32768, 128,
                               "bf16", True)

PREFILL_WORKLOADS = {1: CFG1, 2: CFG2, 3: CFG3}
DECODE_WORKLOADS = {4: CFG4, "5_hkv32": cfg5(32), "5_hkv8": cfg5(8), "5_hkv1": cfg5(1)}


def prefill_inputs(w: PrefillWorkload):
    """(q, k, v) arrays of the workload: q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d]."""
    q = normal([w.seed, STREAM_Q], (w.B, w.Hq, w.Sq, w.d), w.dtype)
    k = normal([w.seed, STREAM_K], (w.B, w.Hkv, w.Sk, w.d), w.dtype)
    v = normal([w.seed, STREAM_V], (w.B, w.Hkv, w.Sk, w.d), w.dtype)
    return q, k, v


def seq_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    rng = np.random.default_rng([seed, STREAM_LENS])
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def block_placement(seed: int, lens: np.ndarray, max_blocks: int,
                    block_size: int = BLOCK_SIZE, spare_blocks: int = 0):
    """Random physical placement of each sequence's logical blocks.

    Logical blocks (b, j), j < ceil(L_b / block_size), enumerated b-major, get
    physical ids ``rng.permutation(num_blocks)``.  Returns (block_table int32
    [B, max_blocks] with -1 in unused entries, num_blocks).  ``spare_blocks``
    extra physical blocks are allocated and never referenced.
    """
    lens = np.asarray(lens, dtype=np.int64)
    nblk = -(-lens // block_size)
    if (nblk > max_blocks).any():
        raise ValueError("a sequence needs more blocks than max_blocks")
    total = int(nblk.sum())
    num_blocks = total + spare_blocks
    rng = np.random.default_rng([seed, STREAM_PERM])
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((len(lens), max_blocks), -1, np.int32)
    pos = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[pos:pos + n]
        pos += int(n)
    return table, max(num_blocks, 1)


@dataclass
class DecodeInputs:
    q: np.ndarray                 # [B, Hq, d]
    k_cache: np.ndarray           # contiguous [B, Hkv, S_max, d] or paged [N, Hkv, 16, d]
    v_cache: np.ndarray
    seq_lens: np.ndarray          # int32 [B]
    block_table: Optional[np.ndarray] = None   # int32 [B, max_blocks] (paged only)
    num_blocks: int = 0
    max_seq_len: int = 0
    extra: dict = field(default_factory=dict)


def decode_inputs(w: DecodeWorkload, lens: Optional[np.ndarray] = None) -> DecodeInputs:
    """Inputs of a decode workload; ``lens`` overrides the drawn lengths."""
    if lens is None:
        lens = seq_lengths(w.seed, w.B, w.L_lo, w.L_hi)
    lens = np.asarray(lens, np.int32)
    q = normal([w.seed, STREAM_Q], (w.B, w.Hq, w.d), w.dtype)
    if w.paged:
        table, nb = block_placement(w.seed, lens, w.max_blocks)
        shape = (nb, w.Hkv, BLOCK_SIZE, w.d)
        k = normal([w.seed, STREAM_K], shape, w.dtype)
        v = normal([w.seed, STREAM_V], shape, w.dtype)
        return DecodeInputs(q, k, v, lens, table, nb, w.max_blocks * BLOCK_SIZE)
    shape = (w.B, w.Hkv, w.S_max, w.d)
    k = normal([w.seed, STREAM_K], shape, w.dtype)
    v = normal([w.seed, STREAM_V], shape, w.dtype)
    return DecodeInputs(q, k, v, lens, None, 0, w.S_max)


def decode_kv_bytes(lens, Hkv: int, d: int, elem_bytes: int = 2) -> int:
    """Algorithmic decode traffic: every cached K and V element read once."""
    return int(np.asarray(lens, np.int64).sum()) * 2 * Hkv * d * elem_bytes
