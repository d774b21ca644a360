"""fp64 CPU oracle for exact scaled-dot-product attention with grouped K/V heads.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package.  The GPU library never
calls it, shares no code with it, and nothing here imports the GPU library.

Sources (the web pages the method is taken from):

* [Different attention mechanisms, §1 MHA, step 3] per head,
  Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V.
* [Attention variants deep-dive, §5 GQA code] softmax subtracts the row
  maximum before ``exp``; query heads must be a multiple of K/V heads; the
  default scale is 1/sqrt(d_head); each K/V head is repeated ``group_size``
  times along the head axis, i.e. query head h reads K/V head floor(h/g).
* [Different attention mechanisms, §3 GQA] every N/G query heads share one
  K/V pair; [§2 MQA] with one K/V head all query heads read it.
* [Attention variants deep-dive, §6.2 forward pseudocode] the tiled online
  softmax; the pages state it gives exactly the one-shot result.
* [Different attention mechanisms, §5 Page Attention, steps 1-2] fixed-size
  KV blocks stored non-contiguously and a per-sequence page table mapping
  logical to physical blocks.
* [Generative AI dev course, MHA/GQA/MQA section] and [Attention variants
  deep-dive, §7 KV Cache] the KV-cache size formula.

Readings where the pages are silent (each is listed in the design notes):

* causal mask: key j is visible to query i iff j <= i + (Sk - Sq)
  (bottom-right alignment; j <= i when Sq == Sk);
* decode: the single new query attends every cached key [0, L_b) unmasked;
  L_b == 0 gives a zero output and LSE = -inf;
* paged decode: logical token t of sequence b lives in physical block
  block_table[b][t // block_size], slot t % block_size.

The main functions materialise the full score matrix on purpose: that is the
plain definition, which the tiled GPU kernels must reproduce.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ----------------------------------------------------------------------------
# input decoding (the oracle's own; exact)
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def to_f64(x, dtype: str) -> np.ndarray:
    """Upcast stored inputs exactly: float32 values, or bfloat16 bit patterns."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# the definition
# ----------------------------------------------------------------------------
def default_scale(d_head: int) -> float:
    """1/sqrt(d_head) [Attention variants deep-dive, §5 GQA code]."""
    return 1.0 / math.sqrt(d_head)


def kv_head_index(hq: int, num_q_heads: int, num_kv_heads: int) -> int:
    """K/V head read by query head ``hq``.

    Query heads form contiguous groups of g = Hq / Hkv that share one K/V head
    [Different attention mechanisms, §3 GQA]; repeating each K/V head g times
    along the head axis [Attention variants deep-dive, §5 GQA code] puts K/V
    head floor(hq / g) under query head hq.
    """
    if num_kv_heads <= 0 or num_q_heads % num_kv_heads != 0:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    return hq // (num_q_heads // num_kv_heads)


def causal_visible(rows: np.ndarray, Sq: int, Sk: int) -> np.ndarray:
    """Boolean [len(rows), Sk]: key j visible to query row i iff j <= i + Sk - Sq."""
    j = np.arange(Sk)[None, :]
    return j <= (np.asarray(rows)[:, None] + (Sk - Sq))


def window_visible(rows: np.ndarray, Sq: int, Sk: int, window: int) -> np.ndarray:
    """Boolean [len(rows), Sk]: sliding window of ``window`` keys ending at the
    causal diagonal, key j visible to row i iff i + Sk - Sq - window < j <= i + Sk - Sq.

    The pages only name sliding-window attention for long sequences
    [Attention variants deep-dive, §8 Q4]; the reading: each query sees its
    last ``window`` keys (itself included), causal.
    """
    j = np.arange(Sk)[None, :]
    last = np.asarray(rows)[:, None] + (Sk - Sq)
    return (j <= last) & (j > last - window)


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool = False, rows=None, window=None):
    """Attention of one query head over one K/V head, in float64.

    q [Sq, d], k [Sk, d], v [Sk, d].  ``rows`` selects query rows (default:
    all).  ``window`` (>= 1) restricts each row to its last ``window`` keys
    and implies causal.  Returns (o [R, d], lse [R], p [R, Sk]): the output,
    the natural-log normaliser m + ln(l), and the probability matrix.
    Rows with no visible key give o = 0 and lse = -inf.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Sq, Sk = q.shape[0], k.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    R, dv = len(rows), v.shape[1]
    if Sk == 0 or R == 0:
        return np.zeros((R, dv)), np.full(R, NEG_INF), np.zeros((R, Sk))
    s = (q[rows] @ k.T) * scale                       # scores, [R, Sk]
    if window is not None:
        s = np.where(window_visible(rows, Sq, Sk, window), s, NEG_INF)
    elif causal:
        s = np.where(causal_visible(rows, Sq, Sk), s, NEG_INF)
    m = s.max(axis=1, keepdims=True)                  # row max (stable softmax)
    empty = ~np.isfinite(m[:, 0])
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    l = e.sum(axis=1, keepdims=True)
    l_safe = np.where(l > 0, l, 1.0)
    p = e / l_safe
    o = p @ v
    lse = m[:, 0] + np.log(l_safe[:, 0])
    o[empty] = 0.0
    lse[empty] = NEG_INF
    return o, lse, p


def attention(q, k, v, scale=None, causal=False, return_lse=False, window=None):
    """Grouped-query attention, q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] -> o [B,Hq,Sq,d].

    MHA when Hkv == Hq, MQA when Hkv == 1 [Attention variants deep-dive, §4 GQA].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if Bk != B or dk != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("shape mismatch")
    if (causal or window is not None) and Sq > Sk:
        raise ValueError("causal attention needs Sq <= Sk")
    if scale is None:
        scale = default_scale(d)
    o = np.zeros((B, Hq, Sq, v.shape[3]))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_index(hq, Hq, Hkv)
            o[b, hq], lse[b, hq], _ = attention_head(q[b, hq], k[b, hk], v[b, hk], scale, causal, window=window)
    return (o, lse) if return_lse else o


def attention_rows(q, k, v, b: int, hq: int, rows, scale=None, causal=False, window=None):
    """Selected output rows of query head ``hq`` in batch ``b`` (for sampled checks)."""
    B, Hq, Sq, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = default_scale(d)
    hk = kv_head_index(hq, Hq, Hkv)
    o, lse, _ = attention_head(np.asarray(q[b, hq], np.float64), np.asarray(k[b, hk], np.float64),
                               np.asarray(v[b, hk], np.float64), scale, causal, rows, window)
    return o, lse


# ----------------------------------------------------------------------------
# decode over a KV cache
# ----------------------------------------------------------------------------
def decode_key_range(L: int, window=None):
    """Keys [lo, hi) the new query of a sequence of cached length L attends.

    All cached keys [0, L) [Attention variants deep-dive, §7 KV Cache]; with a
    sliding window of W keys only the last W of them, [max(0, L - W), L)
    (the window reading of :func:`window_visible` at the newest position).
    """
    if window is None:
        return 0, L
    return max(0, L - window), L


def decode_contiguous(q, k_cache, v_cache, seq_lens, scale=None, heads=None, return_lse=False, window=None):
    """One new query token per sequence over a contiguous cache.

    q [B,Hq,d]; k_cache/v_cache [B,Hkv,S_max,d]; seq_lens [B].  Query b attends
    cached keys [0, L_b) with no mask [Attention variants deep-dive, §7 KV
    Cache: each step only the new token's Q against the cached K/V].
    ``heads`` optionally restricts the work to a list of (b, hq) pairs (others
    are left zero).  ``window``: the query attends only keys
    [max(0, L_b - window), L_b) (its last ``window`` tokens).
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    if scale is None:
        scale = default_scale(d)
    o = np.zeros((B, Hq, v_cache.shape[3]))
    lse = np.full((B, Hq), NEG_INF)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, hq in pairs:
        L = int(seq_lens[b])
        lo, hi = decode_key_range(L, window)
        hk = kv_head_index(hq, Hq, Hkv)
        kb = np.asarray(k_cache[b, hk, lo:hi], np.float64)
        vb = np.asarray(v_cache[b, hk, lo:hi], np.float64)
        ob, lb, _ = attention_head(np.asarray(q[b, hq], np.float64)[None, :], kb, vb, scale)
        o[b, hq], lse[b, hq] = ob[0], lb[0]
    return (o, lse) if return_lse else o


def paged_logical_rows(pages, block_table_row, hk: int, L: int, block_size: int = 16):
    """Logical rows [0, L) of K/V head ``hk`` gathered through one page-table row.

    pages [num_blocks, Hkv, block_size, d]; token t lives in physical block
    block_table_row[t // block_size] at slot t % block_size
    [Different attention mechanisms, §5 Page Attention, steps 1-2].
    """
    t = np.arange(L, dtype=np.int64)
    phys = np.asarray(block_table_row, dtype=np.int64)[t // block_size]
    if L and (phys.min() < 0 or phys.max() >= pages.shape[0]):
        raise IndexError("block table entry out of range")
    return pages[phys, hk, t % block_size]


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale=None, block_size=16,
                 heads=None, return_lse=False, window=None):
    """Decode over a paged cache: gather the logical K/V rows, then the definition
    (``window`` as in decode_contiguous)."""
    B, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    if scale is None:
        scale = default_scale(d)
    o = np.zeros((B, Hq, v_pages.shape[3]))
    lse = np.full((B, Hq), NEG_INF)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    cache = {}
    for b, hq in pairs:
        L = int(seq_lens[b])
        hk = kv_head_index(hq, Hq, Hkv)
        if (b, hk) not in cache:
            cache.clear()
            cache[(b, hk)] = (
                np.asarray(paged_logical_rows(k_pages, block_table[b], hk, L, block_size), np.float64),
                np.asarray(paged_logical_rows(v_pages, block_table[b], hk, L, block_size), np.float64))
        kb, vb = cache[(b, hk)]
        lo, hi = decode_key_range(L, window)
        ob, lb, _ = attention_head(np.asarray(q[b, hq], np.float64)[None, :], kb[lo:hi], vb[lo:hi], scale)
        o[b, hq], lse[b, hq] = ob[0], lb[0]
    return (o, lse) if return_lse else o


# ----------------------------------------------------------------------------
# KV-cache size
# ----------------------------------------------------------------------------
def kv_cache_bytes(seq_len: int, num_kv_heads: int, d_head: int, batch: int = 1,
                   bytes_per_elem: int = 2, num_layers: int = 1) -> int:
    """2 (K and V) x L x Hkv x d_head x batch x bytes, per layer, times layers.

    [Generative AI dev course, MHA/GQA/MQA section] gives the per-layer form
    with batch; [Attention variants deep-dive, §7 KV Cache] the per-model form
    with layers.
    """
    return 2 * seq_len * num_kv_heads * d_head * batch * bytes_per_elem * num_layers


# ----------------------------------------------------------------------------
# the tiled algorithm (used only to pin the pages' equivalence claim)
# ----------------------------------------------------------------------------
def softmax_state(q_rows, k_blk, v_blk, scale, visible):
    """Softmax summary of one block of keys for a set of query rows.

    Returns (m, l, acc): per row the largest visible score m, the sum
    l = sum_j exp(s_j - m) and the unnormalised sum acc = sum_j exp(s_j - m) v_j
    over the block's visible keys.  A row that sees no key of the block gets
    the empty summary (-inf, 0, 0).  The pages' block probabilities are read
    as these unnormalised exp(s - m) [Attention variants deep-dive, §6.2].
    """
    s = np.where(visible, (q_rows @ k_blk.T) * scale, NEG_INF)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], NEG_INF)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.where(visible, np.exp(s - m_safe[:, None]), 0.0)
    return m, e.sum(axis=1), e @ v_blk


def merge_softmax_states(x, y):
    """Combine the summaries of two disjoint key sets into the summary of their union.

    Both are re-expressed against the larger maximum M: each summary's l and
    acc are multiplied by exp(m - M), then added.  This is the rescaling step
    of the online softmax [Attention variants deep-dive, §6.2 (running max and
    sum corrected by exp of the max difference); Different attention
    mechanisms, §4 (online softmax)]; the merge is associative and the empty
    summary is its identity.
    """
    (mx, lx, ax), (my, ly, ay) = x, y
    M = np.maximum(mx, my)
    M_safe = np.where(np.isfinite(M), M, 0.0)
    wx = np.where(np.isfinite(mx), np.exp(mx - M_safe), 0.0)
    wy = np.where(np.isfinite(my), np.exp(my - M_safe), 0.0)
    return M, wx * lx + wy * ly, wx[:, None] * ax + wy[:, None] * ay


def tiled_forward(q, k, v, scale, block_q: int, block_k: int, causal=False, window=None):
    """One head of attention computed tile by tile, in float64.

    Query rows are taken block_q at a time; for each query block the key/value
    blocks of block_k keys are summarised with :func:`softmax_state` and folded
    left to right into a running summary with :func:`merge_softmax_states`;
    the output is acc / l.  No score matrix wider than one key block exists at
    any time, which is what the pages' tiling achieves [Attention variants
    deep-dive, §6.2; Different attention mechanisms, §4]; the pages state the
    result is exactly the one-shot softmax.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Sq, Sk = q.shape[0], k.shape[0]
    o = np.zeros((Sq, v.shape[1]))
    for i0 in range(0, Sq, block_q):
        rows = np.arange(i0, min(Sq, i0 + block_q))
        run = (np.full(len(rows), NEG_INF), np.zeros(len(rows)), np.zeros((len(rows), v.shape[1])))
        for j0 in range(0, Sk, block_k):
            cols = np.arange(j0, min(Sk, j0 + block_k))
            if window is not None:
                vis = window_visible(rows, Sq, Sk, window)[:, cols]
            elif causal:
                vis = causal_visible(rows, Sq, Sk)[:, cols]
            else:
                vis = np.ones((len(rows), len(cols)), dtype=bool)
            run = merge_softmax_states(run, softmax_state(q[rows], k[cols], v[cols], scale, vis))
        _, l, acc = run
        o[rows] = acc / np.where(l > 0, l, 1.0)[:, None]
    return o


def split_partials(q_row, k, v, scale, split_size: int):
    """Partial results over consecutive key splits of one query row.

    Each split s yields (o_s, lse_s): attention restricted to that split's keys
    and its log normaliser.  Their merge (:func:`combine_partials`) is the
    rescale step of the tiled loop applied across splits.
    """
    parts = []
    for j0 in range(0, k.shape[0], split_size):
        o, lse, _ = attention_head(np.asarray(q_row, np.float64)[None, :], k[j0:j0 + split_size],
                                   v[j0:j0 + split_size], scale)
        parts.append((o[0], lse[0]))
    return parts


def combine_partials(parts):
    """Merge (o_s, lse_s) pairs: weights exp(lse_s - max lse), normalised."""
    if not parts:
        raise ValueError("no partials")
    lses = np.array([p[1] for p in parts])
    M = lses.max()
    if not np.isfinite(M):
        return np.zeros_like(parts[0][0]), NEG_INF
    w = np.exp(lses - M)
    o = sum(wi * p[0] for wi, p in zip(w, parts)) / w.sum()
    return o, M + np.log(w.sum())
