"""Planted mistakes in the oracle (CPU only) must each fail at least one pin.

Every mutant below is a plausible slip in writing the definition: a dropped
scale, a wrong softmax axis, a wrong head mapping, a causal off-by-one, a
wrong mask alignment, a missing normalisation, a wrong LSE, a swapped page
index.  Each is patched into ``oracle.core`` for the duration of one test and
the pins of ``test_oracle`` are run against it; at least one must fail.
"""
import numpy as np
import pytest

from oracle import core as A
import tests.test_oracle as P

NEG_INF = -np.inf


def _head(scale_mode="mul", axis=1, causal_mode="br", normalise=True, lse_mode="log", sub_max=True):
    def attention_head(q, k, v, scale, causal=False, rows=None):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        Sq, Sk = q.shape[0], k.shape[0]
        rows = np.arange(Sq) if rows is None else np.asarray(rows)
        if Sk == 0 or len(rows) == 0:
            return np.zeros((len(rows), v.shape[1])), np.full(len(rows), NEG_INF), np.zeros((len(rows), Sk))
        s = q[rows] @ k.T
        s = s * scale if scale_mode == "mul" else (s / scale if scale_mode == "div" else s)
        if causal:
            j = np.arange(Sk)[None, :]
            i = rows[:, None]
            vis = {"br": j <= i + Sk - Sq, "tl": j <= i, "off1": j < i + Sk - Sq}[causal_mode]
            if causal_mode == "off1":
                vis = vis | ((j == 0) & (i == 0))
            s = np.where(vis, s, NEG_INF)
        m = s.max(axis=axis, keepdims=True)
        e = np.exp(s - m) if sub_max else np.exp(s)
        l = e.sum(axis=axis, keepdims=True)
        p = e / l if normalise else e
        o = p @ v
        lse = (m + np.log(l)) if lse_mode == "log" else (m + l)
        lse = lse[:, 0] if axis == 1 else np.broadcast_to(lse, s.shape)[:, 0]
        return o, lse, p
    return attention_head


def _wrong_kv_head(hq, Hq, Hkv):
    if Hq % Hkv:
        raise ValueError
    return hq % Hkv


def _swapped_pages(pages, row, hk, L, block_size=16):
    t = np.arange(L)
    return pages[np.asarray(row)[t % block_size], hk, t // block_size]


MUTANTS = {
    "scale_dropped": ("attention_head", _head(scale_mode="none")),
    "scale_divides": ("attention_head", _head(scale_mode="div")),
    "softmax_over_queries": ("attention_head", _head(axis=0)),
    "causal_top_left": ("attention_head", _head(causal_mode="tl")),
    "causal_off_by_one": ("attention_head", _head(causal_mode="off1")),
    "no_normalisation": ("attention_head", _head(normalise=False)),
    "lse_without_log": ("attention_head", _head(lse_mode="lin")),
    "no_max_subtraction": ("attention_head", _head(sub_max=False)),
    "interleaved_heads": ("kv_head_index", _wrong_kv_head),
    "page_index_swapped": ("paged_logical_rows", _swapped_pages),
}

PINS = [
    (P.test_hand_example_two_keys, ()),
    (P.test_hand_example_scale_multiplies_scores, ()),
    (P.test_hand_example_three_keys_with_mask, ()),
    (P.test_single_key_returns_its_value_row_exactly, ()),
    (P.test_equal_scores_give_mean_of_values, ()),
    (P.test_causal_square_row_i_sees_keys_up_to_i, ()),
    (P.test_probability_rows_sum_to_one, ()),
    (P.test_lse_is_log_of_normaliser, ()),
    (P.test_softmax_shift_invariance_large_scores, ()),
    (P.test_matches_brute_force, (4, 2, True)),
    (P.test_matches_brute_force, (6, 3, False)),
    (P.test_matches_torch_sdpa_float64, (4, 2, True)),
    (P.test_split_partials_combine_to_one_pass, (16,)),
    (P.test_paged_gather_matches_explicit_loops, ()),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(A, attr, fn)
    failed = []
    for pin, args in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(*args)
        except Exception:          # an assertion or a crash both count as caught
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    for pin, args in PINS:
        pin(*args)
