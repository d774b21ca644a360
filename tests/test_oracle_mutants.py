"""Planted mistakes in the oracle (CPU only) must each fail at least one pin.

Every mutant below is a plausible slip in writing the definition or one of
the oracle's helpers: a dropped scale, a wrong softmax axis, a wrong head
mapping, a causal off-by-one, a wrong mask alignment, a row masked by its
place in a selection, a missing normalisation, a wrong LSE, a swapped page
index, a shifted or unclamped decode window, a wrong merge of partial
results, a missing rescale in the tiled loop, and dropped or misplaced terms
of the backward.  Each is patched into the oracle for the duration of one
test and the pins are run against it.  A mutant is caught only when a pin
fails an assertion; any other exception (a crash, a wrong signature) fails
this test, so a mutant that no pin detects cannot hide behind an error.
"""
import numpy as np
import pytest

from oracle import backward as BW
from oracle import core as A
import tests.test_oracle as P
import tests.test_oracle_backward as PB
import tests.test_oracle_window as PW

NEG_INF = -np.inf


def _head(scale_mode="mul", axis=1, causal_mode="br", normalise=True, lse_mode="log", sub_max=True,
          row_index="true"):
    """A rewrite of attention_head with one slip chosen by the arguments."""
    def attention_head(q, k, v, scale, causal=False, rows=None, window=None):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        Sq, Sk = q.shape[0], k.shape[0]
        rows = np.arange(Sq) if rows is None else np.asarray(rows)
        if Sk == 0 or len(rows) == 0:
            return np.zeros((len(rows), v.shape[1])), np.full(len(rows), NEG_INF), np.zeros((len(rows), Sk))
        s = q[rows] @ k.T
        s = s * scale if scale_mode == "mul" else (s / scale if scale_mode == "div" else s)
        j = np.arange(Sk)[None, :]
        i = (rows if row_index == "true" else np.arange(len(rows)))[:, None]
        if window is not None:
            last = i + Sk - Sq
            s = np.where((j <= last) & (j > last - window), s, NEG_INF)
        elif causal:
            vis = {"br": j <= i + Sk - Sq, "tl": j <= i, "off1": j < i + Sk - Sq}[causal_mode]
            if causal_mode == "off1":
                vis = vis | (j == 0)
            s = np.where(vis, s, NEG_INF)
        m = s.max(axis=axis, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m) if sub_max else np.exp(s)
        l = e.sum(axis=axis, keepdims=True)
        p = e / np.where(l > 0, l, 1.0) if normalise else e
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


def _decode_range(mode):
    def decode_key_range(L, window=None):
        if window is None:
            return 0, L
        if mode == "off_by_one":
            return max(0, L - window + 1), L
        return L - window, L          # "unclamped": a negative start wraps around
    return decode_key_range


def _combine(mode):
    def combine_partials(parts):
        lses = np.array([p[1] for p in parts])
        M = lses.max()
        if not np.isfinite(M):
            return np.zeros_like(parts[0][0]), NEG_INF
        w = np.ones_like(lses) if mode == "equal_weights" else np.exp(lses - M)
        o = sum(wi * p[0] for wi, p in zip(w, parts)) / w.sum()
        lse = M + np.log(w.sum()) if mode == "equal_weights" else M + w.sum()
        return o, lse
    return combine_partials


def _merge(mode):
    def merge_softmax_states(x, y):
        (mx, lx, ax), (my, ly, ay) = x, y
        M = np.maximum(mx, my)
        M_safe = np.where(np.isfinite(M), M, 0.0)
        wx = np.where(np.isfinite(mx), np.exp(mx - M_safe), 0.0)
        wy = np.where(np.isfinite(my), np.exp(my - M_safe), 0.0)
        if mode == "running_not_rescaled":
            wx = np.where(np.isfinite(mx), 1.0, 0.0)
        if mode == "sum_not_rescaled":
            return M, lx + ly, wx[:, None] * ax + wy[:, None] * ay
        return M, wx * lx + wy * ly, wx[:, None] * ax + wy[:, None] * ay
    return merge_softmax_states


def _backward(mode):
    """attention_backward with one slip."""
    def attention_backward(q, k, v, do, scale=None, causal=False, window=None):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        B, Hq, Sq, d = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        scale = A.default_scale(d) if scale is None else scale
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                hk = A.kv_head_index(h, Hq, Hkv)
                Pm = BW._probabilities(q[b, h], k[b, hk], scale, causal, window, Sq, Sk)
                dv[b, hk] += Pm.T @ do[b, h]
                dP = do[b, h] @ v[b, hk].T
                D = 0.0 if mode == "D_dropped" else (Pm * dP).sum(axis=1, keepdims=True)
                dS = Pm * (dP - D)
                dq[b, h] = (1.0 if mode == "dq_unscaled" else scale) * dS @ k[b, hk]
                if mode == "dk_not_summed":
                    dk[b, hk] = scale * dS.T @ q[b, h]
                elif mode == "dk_from_dP":
                    dk[b, hk] += scale * (Pm * dP).T @ q[b, h]
                else:
                    dk[b, hk] += scale * dS.T @ q[b, h]
        return dq, dk, dv
    return attention_backward


def _sampled_dv_not_summed():
    orig = BW.attention_backward_sampled

    def attention_backward_sampled(q, k, v, do, b, hk, rows, keys, scale=None, causal=False, window=None,
                                   magnitudes=False):
        # keeps only the last head of the group in dv
        Hq, Hkv = q.shape[1], k.shape[1]
        g = Hq // Hkv
        out = orig(q, k, v, do, b, hk, rows, keys, scale, causal, window, magnitudes)
        single = orig(q[:, hk * g + g - 1:hk * g + g], k[:, hk:hk + 1], v[:, hk:hk + 1],
                      do[:, hk * g + g - 1:hk * g + g], b, 0, rows, keys, scale, causal, window, magnitudes)
        return (out[0], out[1], single[2]) + tuple(out[3:])
    return attention_backward_sampled


MUTANTS = {
    "scale_dropped": (A, "attention_head", _head(scale_mode="none")),
    "scale_divides": (A, "attention_head", _head(scale_mode="div")),
    "softmax_over_queries": (A, "attention_head", _head(axis=0)),
    "causal_top_left": (A, "attention_head", _head(causal_mode="tl")),
    "causal_off_by_one": (A, "attention_head", _head(causal_mode="off1")),
    "rows_masked_by_position_in_selection": (A, "attention_head", _head(row_index="position")),
    "no_normalisation": (A, "attention_head", _head(normalise=False)),
    "lse_without_log": (A, "attention_head", _head(lse_mode="lin")),
    "no_max_subtraction": (A, "attention_head", _head(sub_max=False)),
    "interleaved_heads": (A, "kv_head_index", _wrong_kv_head),
    "page_index_swapped": (A, "paged_logical_rows", _swapped_pages),
    "decode_window_off_by_one": (A, "decode_key_range", _decode_range("off_by_one")),
    "decode_window_unclamped": (A, "decode_key_range", _decode_range("unclamped")),
    "combine_equal_weights": (A, "combine_partials", _combine("equal_weights")),
    "combine_lse_without_log": (A, "combine_partials", _combine("lse_without_log")),
    "tiled_running_not_rescaled": (A, "merge_softmax_states", _merge("running_not_rescaled")),
    "tiled_sum_not_rescaled": (A, "merge_softmax_states", _merge("sum_not_rescaled")),
    "backward_D_dropped": (BW, "attention_backward", _backward("D_dropped")),
    "backward_dq_unscaled": (BW, "attention_backward", _backward("dq_unscaled")),
    "backward_dk_not_summed_over_group": (BW, "attention_backward", _backward("dk_not_summed")),
    "backward_dk_from_dP": (BW, "attention_backward", _backward("dk_from_dP")),
    "backward_sampled_dv_one_head": (BW, "attention_backward_sampled", _sampled_dv_not_summed()),
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
    (P.test_selected_rows_match_brute_force, (7, 12, True, None)),
    (P.test_selected_rows_match_brute_force, (6, 11, False, 3)),
    (P.test_merge_of_block_summaries_is_the_summary_of_the_union, ()),
    (P.test_tiled_online_softmax_equals_one_shot, (True, 5, 7)),
    (P.test_split_partials_combine_to_one_pass, (16,)),
    (P.test_paged_gather_matches_explicit_loops, ()),
    (P.test_decode_single_and_empty_sequence, ()),
    (PW.test_window_equals_attention_on_the_explicit_key_slice, (33, 97, 20)),
    (PW.test_decode_window_is_decode_over_the_last_tokens, ()),
    (PB.test_gradients_match_central_differences, (True, None, 3, 7)),
    (PB.test_gradients_match_torch_autograd, (True,)),
    (PB.test_softmax_gradient_identities, ()),
    (PB.test_sampled_backward_agrees_with_the_full_one, (True, 5)),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    module, attr, fn = MUTANTS[name]
    assert hasattr(module, attr), attr
    monkeypatch.setattr(module, attr, fn)
    failed = []
    for pin, args in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(*args)
        except (AssertionError, pytest.fail.Exception):   # only a failed check counts as a catch
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_every_pin():
    for pin, args in PINS:
        pin(*args)
