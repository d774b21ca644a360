"""Pins of the fp8 KV-cache oracle (CPU): the E4M3 format from its bit fields,
nearest-value rounding with ties to even, saturation, per-row scaling, the
format's error bound, and the pages' 'fp8 halves the cache'."""
import numpy as np
import pytest

import oracle
from oracle import kv_fp8 as F


@pytest.mark.parametrize("code,value", [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
                                        (0x38, 1.0), (0x39, 1.125), (0x40, 2.0), (0x77, 240.0), (0x7E, 448.0),
                                        (0xB8, -1.0), (0xFE, -448.0), (0x80, -0.0)])
def test_e4m3_values_from_bit_fields(code, value):
    assert F.e4m3_value(code) == value
    assert np.signbit(F.e4m3_value(code)) == bool(code & 0x80)


def test_e4m3_table_shape():
    t = F.e4m3_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.isfinite(t).sum() == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == F.E4M3_MAX
    # every value is exactly a bfloat16 (top 16 bits of its fp32 pattern)
    bits = pos.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0) and np.all(pos.astype(np.float32) == pos)


def test_encode_round_trips_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = F.e4m3_table()[codes].astype(np.float32)
    assert np.array_equal(F.e4m3_encode(vals), codes)


def test_midpoints_go_to_the_even_code():
    pos = F.e4m3_table()[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)     # exact in fp32
    got = F.e4m3_encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want)
    # just off the midpoint goes to the nearer side
    up = np.nextafter(mids, np.float32(np.inf))
    assert np.array_equal(F.e4m3_encode(up), lo + 1)


@pytest.mark.parametrize("y,code", [(449.0, 0x7E), (463.9, 0x7E), (1e6, 0x7E), (-1e30, 0xFE), (2.0 ** -10, 0x00),
                                    (3 * 2.0 ** -10, 0x02), (1.5 * 2.0 ** -9, 0x02), (2.0 ** -11, 0x00),
                                    (-2.0 ** -11, 0x80), (1.0625, 0x38), (1.0625001, 0x39)])
def test_encode_special_cases(y, code):
    assert int(F.e4m3_encode(np.float32(y))) == code


def test_encode_is_the_nearest_value_by_brute_force():
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.normal(0, 1, 4000), rng.normal(0, 100, 2000), rng.uniform(-2e-3, 2e-3, 2000)])
    y = y.astype(np.float32)
    got = F.e4m3_encode(y)
    pos = F.e4m3_table()[:0x7F]
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    dist = np.abs(a[:, None] - pos[None, :])
    best = dist.min(axis=1)
    for i in range(len(y)):
        cands = np.flatnonzero(dist[i] == best[i])
        want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert int(got[i]) & 0x7F == want and bool(got[i] & 0x80) == bool(np.signbit(y[i]))


def test_quantize_rows_scale_and_error_bound():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 1, (300, 128)).astype(np.float32)
    x[7] = 0.0
    x[8, 5] = -0.0
    x[9] *= 1e-6                                   # tiny rows keep their relative precision
    codes, scale = F.quantize_rows(x)
    assert scale.dtype == np.float32 and codes.dtype == np.uint8
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scale, (amax / np.float32(448)).astype(np.float32))
    # the largest element of a row becomes +-448
    idx = np.abs(x).argmax(axis=1)
    top = codes[np.arange(300), idx]
    assert np.all((top[amax > 0] & 0x7F) == 0x7E)
    assert scale[7] == 0 and np.all(codes[7] == 0)
    xh = F.dequantize_rows(codes, scale)
    err = np.abs(xh - x.astype(np.float64))
    bound = np.maximum(2.0 ** -4 * np.abs(x.astype(np.float64)), 2.0 ** -10 * scale[:, None].astype(np.float64))
    assert np.all(err <= bound * (1 + 1e-6) + 1e-30)


def test_fp8_halves_the_cache():
    # [Attention variants deep-dive, §7]: fp16 -> fp8 halves the KV cache; scales add 4 B per row
    for L, H, d, b in [(4096, 32, 128, 1), (32768, 8, 128, 1), (1000, 1, 64, 3)]:
        half = oracle.kv_cache_bytes(L, H, d, b) // 2
        assert F.fp8_cache_bytes(L, H, d, b) == half + 2 * L * H * b * 4


# ---- planted mistakes must fail a pin -------------------------------------------

def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float32)
    pos = F.e4m3_table()[:0x7F]
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    hi = np.minimum(np.searchsorted(pos, a), len(pos) - 1)
    lo = np.maximum(hi - 1, 0)
    code = np.where(pos[hi] - a <= a - pos[lo], hi, lo).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def _encode_truncate(y):
    y = np.asarray(y, dtype=np.float32)
    pos = F.e4m3_table()[:0x7F]
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    code = (np.searchsorted(pos, a, side="right") - 1).astype(np.uint8)
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def _value_bias8(code):
    code = int(code) & 0xFF
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return float("nan")
    v = m * 2.0 ** -10 if e == 0 else (1 + m / 8) * 2.0 ** (e - 8)
    return -v if code & 0x80 else v


FP8_MUTANTS = {"ties_away": ("e4m3_encode", _encode_ties_away), "truncate": ("e4m3_encode", _encode_truncate),
               "exponent_bias_8": ("e4m3_value", _value_bias8)}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_fails_a_pin(name, monkeypatch):
    attr, fn = FP8_MUTANTS[name]
    monkeypatch.setattr(F, attr, fn)
    if attr == "e4m3_value":
        monkeypatch.setattr(F, "_POS", F.e4m3_table()[:0x7F])
    pins = [lambda: [test_e4m3_values_from_bit_fields(c, v) for c, v in ((0x01, 2.0 ** -9), (0x38, 1.0), (0x7E, 448.0))],
            test_e4m3_table_shape, test_encode_round_trips_every_code, test_midpoints_go_to_the_even_code,
            test_encode_is_the_nearest_value_by_brute_force, test_quantize_rows_scale_and_error_bound]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"mutant {name} passed every pin"
