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


def row_dot(o, do):
    """D_i = sum_d O_id dO_id per query row (equal to sum_j P_ij dP_ij)."""
    return (np.asarray(o, np.float64) * np.asarray(do, np.float64)).sum(axis=-1)
