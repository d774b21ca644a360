"""Pins of the backward oracle (CPU): central finite differences of the
forward definition, torch's float64 autograd of its SDPA (an independent
library routine), the identities of the softmax gradient, and GQA = MHA on
repeated K/V with the head gradients summed."""
import numpy as np
import pytest

import oracle
from oracle import backward as BW


def rand(shape, seed):
    return np.random.default_rng(seed).normal(0, 1, shape)


def loss(q, k, v, g, scale, causal, window):
    return float((oracle.attention(q, k, v, scale=scale, causal=causal, window=window) * g).sum())


@pytest.mark.parametrize("causal,window,Sq,Sk", [(False, None, 5, 6), (True, None, 6, 6), (True, None, 3, 7),
                                                 (True, 3, 7, 7)])
def test_gradients_match_central_differences(causal, window, Sq, Sk):
    B, Hq, Hkv, d = 1, 4, 2, 3
    q, k, v = rand((B, Hq, Sq, d), 1), rand((B, Hkv, Sk, d), 2), rand((B, Hkv, Sk, d), 3)
    g = rand((B, Hq, Sq, d), 4)
    scale = 0.7
    dq, dk, dv = BW.attention_backward(q, k, v, g, scale, causal, window)
    h = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            fp = loss(q, k, v, g, scale, causal, window)
            x[idx] = old - h
            fm = loss(q, k, v, g, scale, causal, window)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        assert np.allclose(dx, num, rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_torch_autograd(causal):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as Fn
    B, Hq, Hkv, S, d = 2, 8, 2, 33, 16
    q, k, v, g = rand((B, Hq, S, d), 5), rand((B, Hkv, S, d), 6), rand((B, Hkv, S, d), 7), rand((B, Hq, S, d), 8)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = Fn.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.25, enable_gqa=True)
    out.backward(torch.tensor(g))
    dq, dk, dv = BW.attention_backward(q, k, v, g, 0.25, causal)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.allclose(mine, ref.numpy(), rtol=0, atol=1e-11)


def test_softmax_gradient_identities():
    B, Hq, Hkv, S, d = 1, 4, 4, 20, 8
    q, k, v, g = rand((B, Hq, S, d), 9), rand((B, Hkv, S, d), 10), rand((B, Hkv, S, d), 11), rand((B, Hq, S, d), 12)
    dq, dk, dv = BW.attention_backward(q, k, v, g, 0.3, causal=False)
    # rows of dS sum to zero, so dK summed over keys vanishes; rows of P sum to one, so dV summed over keys is
    # dO summed over queries
    assert np.allclose(dk.sum(axis=2), 0, atol=1e-12)
    assert np.allclose(dv.sum(axis=2), g.sum(axis=2), atol=1e-12)
    # D_i = sum_d dO O equals sum_j P dP
    o = oracle.attention(q, k, v, scale=0.3)
    D = BW.row_dot(o, g)
    P = BW._probabilities(q[0, 1], k[0, 1], 0.3, False, None, S, S)
    assert np.allclose(D[0, 1], (P * (g[0, 1] @ v[0, 1].T)).sum(axis=1), atol=1e-12)


def test_gqa_gradients_are_summed_mha_gradients():
    B, Hq, Hkv, S, d = 1, 6, 2, 12, 4
    q, k, v, g = rand((B, Hq, S, d), 13), rand((B, Hkv, S, d), 14), rand((B, Hkv, S, d), 15), rand((B, Hq, S, d), 16)
    dq, dk, dv = BW.attention_backward(q, k, v, g, 0.5, causal=True)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    dq2, dk2, dv2 = BW.attention_backward(q, kr, vr, g, 0.5, causal=True)
    assert np.allclose(dq, dq2, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(B, Hkv, 3, S, d).sum(axis=2), atol=1e-12)
    assert np.allclose(dv, dv2.reshape(B, Hkv, 3, S, d).sum(axis=2), atol=1e-12)


def test_dropped_term_fails_a_pin(monkeypatch):
    def wrong(q, k, v, do, scale=None, causal=False, window=None):
        dq, dk, dv = BW_ORIG(q, k, v, do, scale, causal, window)
        return dq, dk, dv * 0.5 + dk * 0.0
    BW_ORIG = BW.attention_backward

    def no_D(q, k, v, do, scale=None, causal=False, window=None):   # the D term dropped from dS
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        B, Hq, Sq, d = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                hk = oracle.kv_head_index(h, Hq, Hkv)
                P = BW._probabilities(q[b, h], k[b, hk], scale, causal, window, Sq, Sk)
                dv[b, hk] += P.T @ do[b, h]
                dS = P * (do[b, h] @ v[b, hk].T)
                dq[b, h] = scale * dS @ k[b, hk]
                dk[b, hk] += scale * dS.T @ q[b, h]
        return dq, dk, dv
    for mutant in (wrong, no_D):
        monkeypatch.setattr(BW, "attention_backward", mutant)
        with pytest.raises(AssertionError):
            test_gradients_match_central_differences(False, None, 5, 6)


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 5)])
def test_sampled_backward_agrees_with_the_full_one(causal, window):
    """The restricted products pick out exactly the full gradients' entries."""
    rng = np.random.default_rng(11)
    B, Hq, Hkv, Sq, Sk, d = 2, 6, 2, 9, 13, 4
    q = rng.standard_normal((B, Hq, Sq, d))
    k = rng.standard_normal((B, Hkv, Sk, d))
    v = rng.standard_normal((B, Hkv, Sk, d))
    do = rng.standard_normal((B, Hq, Sq, d))
    dq, dk, dv = BW.attention_backward(q, k, v, do, causal=causal, window=window)
    rows, keys = np.array([0, 4, 8]), np.array([1, 6, 12])
    for b in range(B):
        for hk in range(Hkv):
            sq, sk, sv = BW.attention_backward_sampled(q, k, v, do, b, hk, rows, keys, causal=causal,
                                                       window=window)
            assert sorted(sq) == [h for h in range(Hq) if h // 3 == hk]
            for h, got in sq.items():
                np.testing.assert_allclose(got, dq[b, h, rows], atol=1e-12)
            np.testing.assert_allclose(sk, dk[b, hk, keys], atol=1e-12)
            np.testing.assert_allclose(sv, dv[b, hk, keys], atol=1e-12)


def test_gradient_magnitudes_bound_the_gradients_and_match_sampling():
    """|gradient| <= magnitude entrywise (triangle inequality), equality when
    every term is non-negative, and the sampled variant picks the same entries."""
    rng = np.random.default_rng(12)
    B, Hq, Hkv, Sq, Sk, d = 1, 4, 2, 7, 11, 3
    q = rng.standard_normal((B, Hq, Sq, d))
    k = rng.standard_normal((B, Hkv, Sk, d))
    v = rng.standard_normal((B, Hkv, Sk, d))
    do = rng.standard_normal((B, Hq, Sq, d))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=True)
    mq, mk, mv = oracle.gradient_magnitudes(q, k, v, do, causal=True)
    for g, m in ((dq, mq), (dk, mk), (dv, mv)):
        assert np.all(np.abs(g) <= m + 1e-12)
    # dO >= 0: dv = P^T dO has only non-negative terms
    _, _, dv_pos = oracle.attention_backward(q, k, v, np.abs(do), causal=True)
    _, _, mv_pos = oracle.gradient_magnitudes(q, k, v, np.abs(do), causal=True)
    np.testing.assert_allclose(dv_pos, mv_pos, rtol=1e-12)
    rows, keys = np.array([0, 6]), np.array([2, 10])
    _, _, _, (sq, sk, sv) = oracle.attention_backward_sampled(q, k, v, do, 0, 1, rows, keys, causal=True,
                                                              magnitudes=True)
    for h in (2, 3):
        np.testing.assert_allclose(sq[h], mq[0, h, rows], rtol=1e-12)
    np.testing.assert_allclose(sk, mk[0, 1, keys], rtol=1e-12)
    np.testing.assert_allclose(sv, mv[0, 1, keys], rtol=1e-12)
