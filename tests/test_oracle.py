"""Pins of the fp64 oracle against what the pages and mathematics fix.

None of these compare the oracle with itself: each checks a printed value, a
closed form, an invariant, an independent library routine, or a brute-force
pure-Python evaluation on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import core as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# brute force: scalar Python loops over the definition (tiny inputs only)
# ----------------------------------------------------------------------------
def brute_force_row(q, k, v, b, h, i, Hkv, scale, causal, window=None):
    """One output row by explicit loops, math.exp and math.fsum.

    Query head h of a layer with Hq heads and Hkv K/V heads reads K/V head
    h // (Hq // Hkv).  Query i (of Sq, the last Sq of Sk positions) sees key j
    when j <= i + Sk - Sq under a causal mask, and also j > i + Sk - Sq - W
    under a window of W keys.
    """
    Hq, Sq, d = q.shape[1], q.shape[2], q.shape[3]
    Sk = k.shape[2]
    kh = h // (Hq // Hkv)
    last = i + Sk - Sq
    js = [j for j in range(Sk)
          if (window is None or last - window < j <= last) and (window is not None or not causal or j <= last)]
    sc = [scale * math.fsum(float(q[b, h, i, t]) * float(k[b, kh, j, t]) for t in range(d)) for j in js]
    mx = max(sc)
    ex = [math.exp(s - mx) for s in sc]
    den = math.fsum(ex)
    return np.array([math.fsum(e * float(v[b, kh, j, c]) for e, j in zip(ex, js)) / den
                     for c in range(v.shape[3])])


def brute_force(q, k, v, Hkv, scale, causal, window=None):
    """softmax(q.k * scale) v for every (b, h, i), row by row (brute_force_row)."""
    B, Hq, Sq, _ = q.shape
    out = np.zeros((B, Hq, Sq, v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            for i in range(Sq):
                out[b, h, i] = brute_force_row(q, k, v, b, h, i, Hkv, scale, causal, window)
    return out


# ----------------------------------------------------------------------------
# printed values
# ----------------------------------------------------------------------------
def test_kv_cache_bytes_match_printed_values():
    with open(os.path.join(GOLDEN, "kv_cache_bytes.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) == 8
    for c in cases:
        got = oracle.kv_cache_bytes(c["seq_len"], c["num_kv_heads"], c["d_head"], c["batch"],
                                    c["bytes_per_elem"], c["num_layers"])
        assert got == c["bytes"], c["what"]


def test_kv_cache_bytes_scale_linearly_with_batch_and_heads():
    base = oracle.kv_cache_bytes(100, 8, 128, 1, 2)
    assert oracle.kv_cache_bytes(100, 8, 128, 3, 2) == 3 * base
    assert oracle.kv_cache_bytes(100, 32, 128, 1, 2) == 4 * base   # MHA vs GQA-8: 4x
    assert oracle.kv_cache_bytes(100, 1, 128, 1, 2) * 8 == base     # MQA: 1/8 of GQA-8


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def test_hand_example_two_keys():
    # d = 1, scale = 1: scores (0, ln 3) -> p = (1/4, 3/4) -> o = 0.75
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    v = np.array([[0.0], [1.0]])
    o, lse, p = A.attention_head(q, k, v, 1.0)
    assert abs(p[0, 0] - 0.25) < 1e-15 and abs(p[0, 1] - 0.75) < 1e-15
    assert abs(o[0, 0] - 0.75) < 1e-15
    assert abs(lse[0] - math.log(4.0)) < 1e-15        # ln(e^0 + e^ln3)


def test_hand_example_scale_multiplies_scores():
    # scale 0.5, k = (0, 2 ln 3): the same probabilities as above only if the
    # scale multiplies q.k
    q = np.array([[1.0]])
    k = np.array([[0.0], [2.0 * math.log(3.0)]])
    v = np.array([[2.0], [6.0]])
    o, _, _ = A.attention_head(q, k, v, 0.5)
    assert abs(o[0, 0] - (0.25 * 2 + 0.75 * 6)) < 1e-14


def test_hand_example_three_keys_with_mask():
    # causal, Sq = 2, Sk = 3 (bottom-right): row 0 sees keys 0..1, row 1 sees 0..2
    q = np.array([[1.0], [1.0]])
    k = np.array([[0.0], [math.log(2.0)], [math.log(5.0)]])
    v = np.array([[1.0], [10.0], [100.0]])
    o, _, p = A.attention_head(q, k, v, 1.0, causal=True)
    assert np.allclose(p[0], [1 / 3, 2 / 3, 0.0], atol=1e-15, rtol=0)
    assert np.allclose(p[1], [1 / 8, 2 / 8, 5 / 8], atol=1e-15, rtol=0)
    assert abs(o[0, 0] - (1 + 20) / 3) < 1e-13
    assert abs(o[1, 0] - (1 + 20 + 500) / 8) < 1e-13


def test_default_scale_is_inverse_sqrt_dhead():
    assert oracle.default_scale(64) == 0.125
    rng = np.random.default_rng(0)
    q, k, v = rnd(rng, 1, 2, 5, 16), rnd(rng, 1, 2, 7, 16), rnd(rng, 1, 2, 7, 16)
    assert np.array_equal(oracle.attention(q, k, v), oracle.attention(q, k, v, scale=0.25))


def test_single_key_returns_its_value_row_exactly():
    rng = np.random.default_rng(1)
    q, k, v = rnd(rng, 2, 4, 3, 8), rnd(rng, 2, 2, 1, 8), rnd(rng, 2, 2, 1, 8)
    o = oracle.attention(q, k, v)
    for hq in range(4):
        assert np.array_equal(o[:, hq], np.repeat(v[:, hq // 2], 3, axis=1))


def test_equal_scores_give_mean_of_values():
    rng = np.random.default_rng(2)
    Sk, d = 9, 4
    q = np.zeros((1, 1, 5, d))
    k, v = rnd(rng, 1, 1, Sk, d), rnd(rng, 1, 1, Sk, d)
    o = oracle.attention(q, k, v)
    assert np.allclose(o[0, 0], v[0, 0].mean(axis=0), atol=1e-14, rtol=0)
    # causal, Sq = 5 <= Sk = 9: row i sees keys 0 .. i + 4 (bottom-right alignment)
    oc = oracle.attention(q, k, v, causal=True)
    for i in range(5):
        assert np.allclose(oc[0, 0, i], v[0, 0, :i + 5].mean(axis=0), atol=1e-14, rtol=0)


def test_causal_square_row_i_sees_keys_up_to_i():
    rng = np.random.default_rng(3)
    S, d = 6, 3
    q = np.zeros((1, 1, S, d))
    k, v = rnd(rng, 1, 1, S, d), rnd(rng, 1, 1, S, d)
    oc = oracle.attention(q, k, v, causal=True)
    assert np.array_equal(oc[0, 0, 0], v[0, 0, 0])                      # row 0 = V[0] exactly
    for i in range(S):
        assert np.allclose(oc[0, 0, i], v[0, 0, :i + 1].mean(axis=0), atol=1e-14, rtol=0)


def test_causal_row0_is_v0_for_random_queries():
    rng = np.random.default_rng(4)
    q, k, v = rnd(rng, 2, 4, 7, 5), rnd(rng, 2, 2, 7, 5), rnd(rng, 2, 2, 7, 5)
    o = oracle.attention(q, k, v, causal=True)
    for hq in range(4):
        assert np.array_equal(o[:, hq, 0], v[:, hq // 2, 0])


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def test_probability_rows_sum_to_one():
    rng = np.random.default_rng(5)
    for causal in (False, True):
        _, _, p = A.attention_head(rnd(rng, 11, 8) * 3, rnd(rng, 13, 8), rnd(rng, 13, 8), 0.4, causal)
        assert np.all(np.abs(p.sum(axis=1) - 1.0) <= 1e-12)
        assert np.all(p >= 0)


def test_lse_is_log_of_normaliser():
    rng = np.random.default_rng(6)
    q, k, v = rnd(rng, 4, 6), rnd(rng, 10, 6), rnd(rng, 10, 6)
    _, lse, _ = A.attention_head(q, k, v, 0.3)
    direct = np.log(np.exp(0.3 * q @ k.T).sum(axis=1))
    assert np.allclose(lse, direct, atol=1e-12, rtol=0)


def test_linear_in_values():
    rng = np.random.default_rng(7)
    q, k, v = rnd(rng, 1, 4, 6, 5), rnd(rng, 1, 2, 9, 5), rnd(rng, 1, 2, 9, 5)
    a, c = 2.5, rnd(rng, 5)
    for causal in (False, True):
        o1 = oracle.attention(q, k, v, causal=causal)
        o2 = oracle.attention(q, k, a * v + c, causal=causal)
        assert np.allclose(o2, a * o1 + c, atol=1e-12, rtol=0)


def test_key_permutation_invariance():
    rng = np.random.default_rng(8)
    q, k, v = rnd(rng, 2, 4, 5, 6), rnd(rng, 2, 1, 11, 6), rnd(rng, 2, 1, 11, 6)
    perm = rng.permutation(11)
    assert np.allclose(oracle.attention(q, k, v), oracle.attention(q, k[:, :, perm], v[:, :, perm]),
                       atol=1e-13, rtol=0)


def test_softmax_shift_invariance_large_scores():
    # adding a constant to every score of a row changes nothing; huge scores do not overflow
    q = np.array([[1.0]])
    k = np.array([[1000.0], [1000.0 + math.log(3.0)]])
    v = np.array([[0.0], [1.0]])
    o, _, _ = A.attention_head(q, k, v, 1.0)
    assert abs(o[0, 0] - 0.75) < 1e-12


# ----------------------------------------------------------------------------
# head grouping: MHA / GQA / MQA
# ----------------------------------------------------------------------------
def test_head_mapping_is_contiguous_groups():
    assert [oracle.kv_head_index(h, 32, 8) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head_index(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    assert all(oracle.kv_head_index(h, 32, 1) == 0 for h in range(32))
    with pytest.raises(ValueError):
        oracle.kv_head_index(0, 6, 4)
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 6, 2, 4)), np.zeros((1, 4, 2, 4)), np.zeros((1, 4, 2, 4)))


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_on_repeated_kv(causal):
    rng = np.random.default_rng(9)
    Hq, Hkv = 8, 2
    q, k, v = rnd(rng, 2, Hq, 6, 4), rnd(rng, 2, Hkv, 6, 4), rnd(rng, 2, Hkv, 6, 4)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    assert np.array_equal(oracle.attention(q, k, v, causal=causal),
                          oracle.attention(q, kr, vr, causal=causal))


def test_mqa_every_head_reads_kv_head_zero():
    rng = np.random.default_rng(10)
    q, k, v = rnd(rng, 1, 4, 3, 5), rnd(rng, 1, 1, 7, 5), rnd(rng, 1, 1, 7, 5)
    o = oracle.attention(q, k, v)
    for h in range(4):
        single = oracle.attention(q[:, h:h + 1], k, v)
        assert np.array_equal(o[:, h:h + 1], single)


@pytest.mark.parametrize("Hq,Hkv,causal", [(4, 4, False), (4, 2, True), (6, 3, False), (4, 1, True)])
def test_matches_brute_force(Hq, Hkv, causal):
    rng = np.random.default_rng(11)
    q, k, v = rnd(rng, 2, Hq, 4, 3), rnd(rng, 2, Hkv, 5, 3), rnd(rng, 2, Hkv, 5, 3)
    ref = brute_force(q, k, v, Hkv, 0.7, causal)
    assert np.allclose(oracle.attention(q, k, v, scale=0.7, causal=causal), ref, atol=1e-13, rtol=0)


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 2), st.sampled_from([(1, 1), (2, 1), (2, 2), (4, 2), (6, 2), (8, 4)]),
       st.integers(1, 6), st.integers(0, 4), st.sampled_from([1, 2, 4, 8]), st.booleans(),
       st.integers(0, 2 ** 31 - 1))
def test_property_matches_brute_force(B, heads, Sq, extra_k, d, causal, seed):
    Hq, Hkv = heads
    Sk = Sq + extra_k
    rng = np.random.default_rng(seed)
    q, k, v = rnd(rng, B, Hq, Sq, d), rnd(rng, B, Hkv, Sk, d), rnd(rng, B, Hkv, Sk, d)
    scale = float(rng.uniform(0.1, 2.0))
    ref = brute_force(q, k, v, Hkv, scale, causal)
    got = oracle.attention(q, k, v, scale=scale, causal=causal)
    assert np.allclose(got, ref, atol=1e-12, rtol=1e-12)


# ----------------------------------------------------------------------------
# independent library routine: torch CPU float64 SDPA with enable_gqa
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("Hq,Hkv,causal", [(4, 2, False), (4, 2, True), (8, 8, True), (8, 1, False)])
def test_matches_torch_sdpa_float64(Hq, Hkv, causal):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(12)
    S, d = 37, 16
    q, k, v = rnd(rng, 2, Hq, S, d), rnd(rng, 2, Hkv, S, d), rnd(rng, 2, Hkv, S, d * 2)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal,
        scale=0.3, enable_gqa=True).numpy()
    assert np.abs(oracle.attention(q, k, v, scale=0.3, causal=causal) - ref).max() <= 1e-12


# ----------------------------------------------------------------------------
# selected rows (the reference of the sampled full-size checks)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("Sq,Sk,causal,window", [(9, 9, False, None), (7, 12, True, None), (12, 12, True, None),
                                                 (6, 11, False, 3), (10, 10, False, 4), (5, 9, True, 1)])
def test_selected_rows_match_brute_force(Sq, Sk, causal, window):
    # unsorted, repeated and non-contiguous rows of a GQA head (h = 5 reads K/V head 2):
    # every row must be masked by its own index, not by its place in the selection
    rng = np.random.default_rng(20)
    Hq, Hkv, d = 6, 3, 4
    q, k, v = rnd(rng, 2, Hq, Sq, d), rnd(rng, 2, Hkv, Sk, d), rnd(rng, 2, Hkv, Sk, d)
    rows = np.array([Sq - 1, 0, 3, Sq - 1, 1][:max(1, min(5, Sq))]) % Sq
    o, lse = A.attention_rows(q, k, v, 1, 5, rows, scale=0.8, causal=causal, window=window)
    assert o.shape == (len(rows), d) and lse.shape == (len(rows),)
    for r, i in enumerate(rows):
        ref = brute_force_row(q, k, v, 1, 5, int(i), Hkv, 0.8, causal, window)
        assert np.allclose(o[r], ref, atol=1e-13, rtol=0), (i, o[r], ref)


def test_selected_rows_equal_the_full_head():
    rng = np.random.default_rng(21)
    Hq, Hkv, Sq, Sk, d = 8, 2, 40, 53, 6
    q, k, v = rnd(rng, 2, Hq, Sq, d), rnd(rng, 2, Hkv, Sk, d), rnd(rng, 2, Hkv, Sk, d)
    rows = np.array([39, 0, 17, 16, 33, 2])
    for causal, window in ((False, None), (True, None), (True, 7)):
        full, full_lse = oracle.attention(q, k, v, causal=causal, window=window, return_lse=True)
        for b, hq in ((0, 0), (1, 3), (1, 7)):
            o, lse = A.attention_rows(q, k, v, b, hq, rows, causal=causal, window=window)
            assert np.allclose(o, full[b, hq, rows], atol=1e-13, rtol=0)
            assert np.allclose(lse, full_lse[b, hq, rows], atol=1e-13, rtol=0)


# ----------------------------------------------------------------------------
# the pages' algorithm reaches the definition exactly
# ----------------------------------------------------------------------------
def test_merge_of_block_summaries_is_the_summary_of_the_union():
    # the merged (m, l, acc) of two key sets equals the directly computed summary of their
    # union: m the max score, l = sum exp(s - m), acc = sum exp(s - m) v
    rng = np.random.default_rng(22)
    q, k, v = rnd(rng, 3, 5) * 2, rnd(rng, 9, 5), rnd(rng, 9, 5)
    vis = np.ones((3, 9), dtype=bool)
    vis[1, :4] = False                      # row 1 sees nothing of the first set
    a = A.softmax_state(q, k[:4], v[:4], 0.6, vis[:, :4])
    b = A.softmax_state(q, k[4:], v[4:], 0.6, vis[:, 4:])
    m, l, acc = A.merge_softmax_states(a, b)
    s = np.where(vis, 0.6 * q @ k.T, -np.inf)
    m_ref = s.max(axis=1)
    e = np.exp(s - m_ref[:, None])
    assert np.allclose(m, m_ref, atol=1e-13, rtol=0)
    assert np.allclose(l, e.sum(axis=1), atol=1e-13, rtol=0)
    assert np.allclose(acc, e @ v, atol=1e-13, rtol=0)
    assert not np.isfinite(a[0][1]) and a[1][1] == 0 and np.all(a[2][1] == 0)   # empty summary
    # the empty summary is the identity, on either side
    empty = (np.full(3, -np.inf), np.zeros(3), np.zeros((3, 5)))
    for x in (A.merge_softmax_states(empty, b), A.merge_softmax_states(b, empty)):
        assert all(np.array_equal(p, r) for p, r in zip(x, b))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bq,bk", [(1, 1), (3, 3), (16, 16), (64, 64), (5, 7), (64, 29)])
def test_tiled_online_softmax_equals_one_shot(causal, bq, bk):
    rng = np.random.default_rng(13)
    Sq, Sk, d = 29, 29, 8
    q, k, v = rnd(rng, Sq, d) * 2, rnd(rng, Sk, d), rnd(rng, Sk, d)
    ref, _, _ = A.attention_head(q, k, v, 0.5, causal)
    got = A.tiled_forward(q, k, v, 0.5, bq, bk, causal)
    assert np.abs(got - ref).max() <= 1e-12


def test_tiled_online_softmax_rectangular_causal_and_window():
    rng = np.random.default_rng(14)
    q, k, v = rnd(rng, 10, 4) * 3, rnd(rng, 23, 4), rnd(rng, 23, 4)
    ref, _, _ = A.attention_head(q, k, v, 1.1, True)
    for bq, bk in [(1, 23), (4, 6), (10, 1)]:
        assert np.abs(A.tiled_forward(q, k, v, 1.1, bq, bk, True) - ref).max() <= 1e-12
    for W in (1, 5, 30):
        ref_w, _, _ = A.attention_head(q, k, v, 1.1, window=W)
        for bq, bk in [(3, 4), (10, 23), (1, 2)]:
            assert np.abs(A.tiled_forward(q, k, v, 1.1, bq, bk, window=W) - ref_w).max() <= 1e-12


@pytest.mark.parametrize("split", [1, 3, 16, 64, 100])
def test_split_partials_combine_to_one_pass(split):
    rng = np.random.default_rng(15)
    q, k, v = rnd(rng, 8) * 3, rnd(rng, 100, 8), rnd(rng, 100, 8)
    o_ref, lse_ref, _ = A.attention_head(q[None], k, v, 0.35)
    o, lse = A.combine_partials(A.split_partials(q, k, v, 0.35, split))
    assert np.abs(o - o_ref[0]).max() <= 1e-12
    assert abs(lse - lse_ref[0]) <= 1e-12


# ----------------------------------------------------------------------------
# decode and the paged gather
# ----------------------------------------------------------------------------
def test_decode_single_and_empty_sequence():
    rng = np.random.default_rng(16)
    q, kc, vc = rnd(rng, 3, 4, 8), rnd(rng, 3, 2, 5, 8), rnd(rng, 3, 2, 5, 8)
    lens = np.array([1, 0, 5])
    o, lse = oracle.decode_contiguous(q, kc, vc, lens, return_lse=True)
    for hq in range(4):
        assert np.array_equal(o[0, hq], vc[0, hq // 2, 0])
        assert np.all(o[1, hq] == 0) and lse[1, hq] == -np.inf
    ref = oracle.attention(q[2][None, :, None, :], kc[2][None], vc[2][None])[0, :, 0]
    assert np.allclose(o[2], ref, atol=1e-14, rtol=0)


def test_decode_zero_query_is_mean_of_prefix():
    rng = np.random.default_rng(17)
    kc, vc = rnd(rng, 2, 1, 10, 4), rnd(rng, 2, 1, 10, 4)
    lens = np.array([3, 10])
    o = oracle.decode_contiguous(np.zeros((2, 2, 4)), kc, vc, lens)
    assert np.allclose(o[0, 1], vc[0, 0, :3].mean(axis=0), atol=1e-15, rtol=0)
    assert np.allclose(o[1, 0], vc[1, 0].mean(axis=0), atol=1e-15, rtol=0)


def test_paged_gather_matches_explicit_loops():
    rng = np.random.default_rng(18)
    nb, Hkv, bs, d = 7, 2, 4, 3
    pages = rnd(rng, nb, Hkv, bs, d)
    table = np.array([5, 0, 3, -1])
    L = 10
    got = A.paged_logical_rows(pages, table, 1, L, bs)
    for t in range(L):
        blk, slot = divmod(t, bs)
        assert np.array_equal(got[t], pages[table[blk], 1, slot])
    with pytest.raises(IndexError):
        A.paged_logical_rows(pages, np.array([5, 0, -1]), 0, 12, bs)


def test_paged_decode_equals_contiguous_decode():
    rng = np.random.default_rng(19)
    B, Hq, Hkv, d, bs = 3, 4, 2, 8, 16
    lens = np.array([33, 1, 48])
    nblk = -(-lens // bs)
    num_blocks = int(nblk.sum()) + 2
    perm = rng.permutation(num_blocks)
    table = np.full((B, 4), -1)
    pos = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    kp, vp = rnd(rng, num_blocks, Hkv, bs, d), rnd(rng, num_blocks, Hkv, bs, d)
    kc = np.zeros((B, Hkv, 64, d))
    vc = np.zeros((B, Hkv, 64, d))
    for b in range(B):
        for t in range(lens[b]):
            kc[b, :, t] = kp[table[b, t // bs], :, t % bs]
            vc[b, :, t] = vp[table[b, t // bs], :, t % bs]
    q = rnd(rng, B, Hq, d)
    assert np.array_equal(oracle.decode_paged(q, kp, vp, table, lens),
                          oracle.decode_contiguous(q, kc, vc, lens))


# ----------------------------------------------------------------------------
# exact input decoding
# ----------------------------------------------------------------------------
def test_bf16_decoding_is_exact():
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 1 << 16, dtype=np.uint16)
    got = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
