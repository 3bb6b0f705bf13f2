"""Scaled dot-product attention for one new query over cached keys/values (fp64).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Three independent paths:
  * decode_row       -- the definition for one query over L cached positions;
  * full_causal      -- recompute all rows with the causal mask, no cache;
  * cached_decode    -- the naive cached loop: concatenate the new k, v and attend the new q.
and the variants:
  * grouped_decode   -- several query heads attend one shared key/value head (MQA / GQA);
  * window_decode    -- the query attends only the most recent `window` positions (rolling
                        window), with rolling_cached_decode as the page's step-by-step procedure.
"""
from __future__ import annotations

import numpy as np


def decode_row(q, K, V, scale) -> np.ndarray:
    """softmax(scale * q . K^T) . V for one query over L cached positions, in fp64.

    q: [D]; K, V: [L, D] (any real dtype, widened exactly to fp64); scale: a float, used as the
    exact fp64 value of the number passed. Returns [D] fp64.

    The new query attends every cached position, its own included, with no mask: in the cached
    path causality holds by construction ("LLM Inference Acceleration -- KV Cache", section 3.1,
    the Attention class writes the new k/v at start_pos and then reads [0, start_pos+seqlen);
    "From Neuron to GPT -- KV cache chapter", cached attention layer: no causal mask with a
    cache). The softmax is taken in higher precision than the stored values (section 3.1 casts
    the scores to float before the softmax); here fp64.

    L = 0 gives the zero vector (nothing to attend).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = (K @ q) * float(scale)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum()


def full_causal(Q, K, V, scale, start_pos: int = 0) -> np.ndarray:
    """Recompute attention for a chunk of queries against all keys, with the causal mask.

    Q: [T, D] holds queries for positions start_pos .. start_pos+T-1; K, V: [start_pos+T, D].
    Row i may attend positions 0 .. start_pos+i. The mask is the upper-triangular -inf matrix
    with diagonal offset start_pos+1, added to the scaled scores before the row softmax
    ("LLM Inference Acceleration -- KV Cache", section 2.1, the two worked steps; section 3.1,
    Transformer.forward builds triu(-inf, diagonal=start_pos+1) when seqlen > 1).
    Returns [T, D] fp64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    T = Q.shape[0]
    S = K.shape[0]
    if S != start_pos + T:
        raise ValueError("keys must cover every position up to the last query")
    scores = (Q @ K.T) * float(scale)
    mask = np.triu(np.full((T, S), -np.inf), k=start_pos + 1)
    scores = scores + mask
    m = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - m)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def cached_decode(Qs, Ks, Vs, scale, prefix_K=None, prefix_V=None) -> np.ndarray:
    """The naive cached path: for each step, append the new k, v to the cache by concatenation
    and attend the new q over the whole cache.

    Qs, Ks, Vs: [T, D] -- the new token's q, k, v at each of T steps. prefix_K/prefix_V: [P, D]
    entries already cached (optional). Returns [T, D]: the output row of each step.

    Follows "KV Cache Mechanism Explained", section 3.2 (forward_with_cache: concatenate the
    cached K/V with K_new/V_new, store it back, attend Q_new) and section 4 (the cache grows by
    exactly one entry per generated token).
    """
    Qs = np.asarray(Qs, dtype=np.float64)
    D = Qs.shape[1]
    K_cache = np.zeros((0, D)) if prefix_K is None else np.asarray(prefix_K, dtype=np.float64)
    V_cache = np.zeros((0, D)) if prefix_V is None else np.asarray(prefix_V, dtype=np.float64)
    rows = []
    for t in range(Qs.shape[0]):
        K_cache = np.concatenate([K_cache, np.asarray(Ks[t:t + 1], dtype=np.float64)], axis=0)
        V_cache = np.concatenate([V_cache, np.asarray(Vs[t:t + 1], dtype=np.float64)], axis=0)
        rows.append(decode_row(Qs[t], K_cache, V_cache, scale))
    return np.stack(rows) if rows else np.zeros((0, D))


def kv_head_of(hq: int, q_heads: int, kv_heads: int) -> int:
    """The key/value head that query head hq reads when q_heads query heads share kv_heads
    key/value heads.

    "LLM Inference Acceleration -- KV Cache", section 6.2: MHA has one key/value head per query
    head; MQA gives all heads one shared key/value head, each head keeping its own query; GQA
    splits the query heads into groups and each group shares one key/value head. The page does
    not say which query heads form a group; the reading here is consecutive runs of
    G = q_heads / kv_heads heads (query head hq belongs to group hq // G), which makes MHA the
    case G = 1 and MQA the case kv_heads = 1.
    """
    if kv_heads < 1 or q_heads % kv_heads:
        raise ValueError("the query heads must split evenly over the key/value heads")
    return hq // (q_heads // kv_heads)


def grouped_decode(q, K, V, scale) -> np.ndarray:
    """Decode for one sequence with shared key/value heads.

    q: [Hq, D]; K, V: [Hkv, L, D] with Hq a multiple of Hkv. Row hq of the result is
    decode_row(q[hq], K[g], V[g]) for g = kv_head_of(hq, Hq, Hkv). Returns [Hq, D] fp64.
    """
    q = np.asarray(q)
    Hq, Hkv = q.shape[0], K.shape[0]
    return np.stack([decode_row(q[h], K[kv_head_of(h, Hq, Hkv)], V[kv_head_of(h, Hq, Hkv)], scale)
                     for h in range(Hq)])


def window_start(L: int, window: int) -> int:
    """First position attended at attended length L (the new token included) under a rolling
    window of `window` positions; window 0 means no window."""
    if window < 0 or L < 0:
        raise ValueError("window and length must be non-negative")
    return max(0, L - window) if window else 0


def window_decode(q, K, V, scale, window: int) -> np.ndarray:
    """Decode under a rolling window: the new query attends only the most recent `window`
    positions, its own included.

    "KV Cache Mechanism Explained", section 8, item 2: the cache keeps a fixed-size window; when
    it holds more than WINDOW_SIZE entries only the last WINDOW_SIZE are kept. The reading taken:
    the trim follows each append and precedes the attention, so a query at length L attends
    positions window_start(L, window) .. L-1. K, V: [L, D] hold every position 0 .. L-1.
    """
    s = window_start(np.asarray(K).shape[0], window)
    return decode_row(q, np.asarray(K)[s:], np.asarray(V)[s:], scale)


def rolling_cached_decode(Qs, Ks, Vs, scale, window: int) -> np.ndarray:
    """The rolling cache of "KV Cache Mechanism Explained", section 8, item 2, step by step:
    each step concatenates the new k, v onto the cache; if the cache then holds more than
    `window` entries it keeps only the last `window`; the new query attends the whole cache.
    window 0 never trims. Qs, Ks, Vs: [T, D]. Returns [T, D]."""
    Qs = np.asarray(Qs, dtype=np.float64)
    D = Qs.shape[1]
    K_cache, V_cache = np.zeros((0, D)), np.zeros((0, D))
    rows = []
    for t in range(Qs.shape[0]):
        K_cache = np.concatenate([K_cache, np.asarray(Ks[t:t + 1], dtype=np.float64)], axis=0)
        V_cache = np.concatenate([V_cache, np.asarray(Vs[t:t + 1], dtype=np.float64)], axis=0)
        if window and len(K_cache) > window:
            K_cache = K_cache[-window:]
            V_cache = V_cache[-window:]
        rows.append(decode_row(Qs[t], K_cache, V_cache, scale))
    return np.stack(rows) if rows else np.zeros((0, D))
