"""fp64 CPU oracle for the attention backward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
calls it, shares no code with it, and nothing here imports the GPU library.

The pages fix how the backward is organised, not its arithmetic: it keeps no
attention matrix from the forward and recomputes it from the saved Q, K, V,
trading extra computation for memory traffic, so memory drops from O(n^2) to
O(n) [Attention variants deep-dive, §6.2 technique 2 (recomputation); §8,
follow-up questions 2 and 3].  The gradients themselves follow from the
definition O = softmax(S) V, S = scale * Q K^T (masked entries -inf), for a
loss whose gradient with respect to O is dO:

  dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D)  with  D_i = sum_j P_ij dP_ij,
  dQ = scale * dS K,   dK = scale * dS^T Q,

(the softmax Jacobian applied row by row); D_i equals sum_d dO_id O_id.  With
grouped K/V heads the gradients of a K/V head sum over the g query heads that
read it [Attention variants deep-dive, §5 GQA code: each K/V head repeated g
times].  Written as matrices on purpose: the definition, not the tiled
algorithm.
"""
from __future__ import annotations

import numpy as np

from .core import NEG_INF, causal_visible, default_scale, kv_head_index, window_visible


def _probabilities(q, k, scale, causal, window, Sq, Sk):
    s = (q @ k.T) * scale
    rows = np.arange(Sq)
    if window is not None:
        s = np.where(window_visible(rows, Sq, Sk, window), s, NEG_INF)
    elif causal:
        s = np.where(causal_visible(rows, Sq, Sk), s, NEG_INF)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / np.where(l > 0, l, 1.0)


def attention_backward(q, k, v, do, scale=None, causal=False, window=None):
    """Gradients (dq, dk, dv) of attention(q, k, v) for output gradient do.

    q, do [B, Hq, Sq, d]; k, v [B, Hkv, Sk, d]; all fp64 results.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_index(h, Hq, Hkv)
            P = _probabilities(q[b, h], k[b, hk], scale, causal, window, Sq, Sk)
            dv[b, hk] += P.T @ do[b, h]
            dP = do[b, h] @ v[b, hk].T
            D = (P * dP).sum(axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[b, h] = scale * dS @ k[b, hk]
            dk[b, hk] += scale * dS.T @ q[b, h]
    return dq, dk, dv


def gradient_magnitudes(q, k, v, do, scale=None, causal=False, window=None):
    """Sums of the absolute values of the terms behind each gradient entry.

    (mq, mk, mv) with mv = sum_h P^T |dO|, mq = scale A |K|,
    mk = scale sum_h A^T |Q|, where A = P * (|dP| + Dabs) and
    Dabs_i = sum_d |dO_id| |O_id| >= |D_i|, so A bounds |dS| and each of
    its parts.  A computation that perturbs every term by a relative
    e (rounding an operand, recomputing P from a rounded log-sum-exp, forming
    D from a rounded O) changes a gradient entry by at most e times its
    magnitude; the parity tests state their bounds in these units.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    mq = np.zeros_like(q)
    mk = np.zeros_like(k)
    mv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            hk = kv_head_index(h, Hq, Hkv)
            P = _probabilities(q[b, h], k[b, hk], scale, causal, window, Sq, Sk)
            mv[b, hk] += P.T @ np.abs(do[b, h])
            dP = do[b, h] @ v[b, hk].T
            Dabs = (np.abs(do[b, h]) * np.abs(P @ v[b, hk])).sum(axis=1, keepdims=True)
            A = P * (np.abs(dP) + Dabs)
            mq[b, h] = scale * A @ np.abs(k[b, hk])
            mk[b, hk] += scale * A.T @ np.abs(q[b, h])
    return mq, mk, mv


def row_dot(o, do):
    """D_i = sum_d O_id dO_id per query row (equal to sum_j P_ij dP_ij)."""
    return (np.asarray(o, np.float64) * np.asarray(do, np.float64)).sum(axis=-1)


def attention_backward_sampled(q, k, v, do, b, hk, rows, keys, scale=None, causal=False, window=None,
                               magnitudes=False):
    """Selected gradients of one K/V group, from the same definition.

    For batch b and K/V head hk: dq at query rows ``rows`` of every query head
    reading hk ({h: array [len(rows), d]}), and dk, dv at key rows ``keys``
    (arrays [len(keys), d]) summed over those heads.  The probabilities of a
    head are still formed in full (each row's normaliser needs every key);
    only the products are restricted, so large shapes stay affordable.
    q, do [B, Hq, Sq, d] and k, v [B, Hkv, Sk, d] may be any array-likes
    indexable per (b, head) (converted to fp64 one head at a time).
    ``magnitudes``: also return gradient_magnitudes' values at the same
    entries, as a fourth item (mq, mk, mv).
    """
    Hq, Sq, d = q.shape[1], q.shape[2], q.shape[3]
    Hkv, Sk = k.shape[1], k.shape[2]
    if scale is None:
        scale = default_scale(d)
    rows = np.asarray(rows)
    keys = np.asarray(keys)
    kk = np.asarray(k[b, hk], np.float64)
    vv = np.asarray(v[b, hk], np.float64)
    dq, mq = {}, {}
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    mk = np.zeros((len(keys), d))
    mv = np.zeros((len(keys), d))
    for h in range(Hq):
        if kv_head_index(h, Hq, Hkv) != hk:
            continue
        qh = np.asarray(q[b, h], np.float64)
        doh = np.asarray(do[b, h], np.float64)
        P = _probabilities(qh, kk, scale, causal, window, Sq, Sk)
        O = P @ vv
        D = (doh * O).sum(axis=1, keepdims=True)                # rowsum(dO * O)
        Pk = P[:, keys]
        dv += Pk.T @ doh
        dPk = doh @ vv[keys].T
        dSk = Pk * (dPk - D)
        dk += scale * dSk.T @ qh
        Pr = P[rows]
        dPr = doh[rows] @ vv.T
        dSr = Pr * (dPr - D[rows])
        dq[h] = scale * dSr @ kk
        if magnitudes:
            Dabs = (np.abs(doh) * np.abs(O)).sum(axis=1, keepdims=True)
            mv += Pk.T @ np.abs(doh)
            mk += scale * (Pk * (np.abs(dPk) + Dabs)).T @ np.abs(qh)
            mq[h] = scale * (Pr * (np.abs(dPr) + Dabs[rows])) @ np.abs(kk)
    if magnitudes:
        return dq, dk, dv, (mq, mk, mv)
    return dq, dk, dv
