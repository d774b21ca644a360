"""CPU oracle for an fp8 KV cache: E4M3 codes with one fp32 scale per cached row.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
calls it, shares no code with it, and nothing here imports the GPU library.

Sources: [Attention variants deep-dive, §7 KV Cache: among the factors of the
cache size, precision, where fp16 -> fp8 halves it (the remedy: quantising the
KV cache); §8 Q4: quantise the KV cache to fp8 or int4].  The pages name the
precision only.  Readings (each is listed in the design notes):

* format: the OCP 8-bit E4M3 format -- sign bit, 4 exponent bits with bias 7,
  3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9; no
  infinities; S.1111.111 is NaN, so the largest finite magnitude is
  1.75 * 2^8 = 448;
* one fp32 scale per cached row (one token of one K/V head): amax = the row's
  largest |x|, scale = amax / 448 and y = x * (448 / amax), each operation in
  fp32 rounded to nearest even; a row of zeros gets scale 0 and y = x * 0;
* the code of y is the E4M3 value nearest to |y| (magnitudes past 448 take
  448), ties to the code with an even last bit, with the sign bit of y;
* a code stands for decode(code) * scale, and attention over an fp8 cache is
  the definition applied to those values.

Every E4M3 value is exactly a bfloat16, and its product with an fp32 scale is
exact in fp64, so dequantised rows carry no rounding of their own.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The number an E4M3 code stands for, from its bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """Values of all 256 codes (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_POS = e4m3_table()[:0x7F]        # codes 0x00 .. 0x7E: 0 .. 448, increasing


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of each fp32 value y (ties to the even code,
    magnitudes past 448 take 448, the sign bit copied from y)."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y.astype(np.float64)), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")             # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(y)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Rows x [..., d] (fp32 values, e.g. upcast bf16) -> (codes uint8 [..., d], scales fp32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / amax, np.float32(0)).astype(np.float32)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    y = (x * inv[..., None]).astype(np.float32)
    return e4m3_encode(y), scale


def dequantize_rows(codes, scales) -> np.ndarray:
    """The values the cache stands for, in fp64 (exact)."""
    table = e4m3_table()
    return table[np.asarray(codes, dtype=np.uint8)] * np.asarray(scales, dtype=np.float64)[..., None]


def fp8_cache_bytes(seq_len: int, num_kv_heads: int, d_head: int, batch: int = 1) -> int:
    """K and V codes (one byte each) plus one fp32 scale per row, per layer."""
    rows = 2 * seq_len * num_kv_heads * batch
    return rows * d_head + rows * 4
