"""Pins for the rolling-window oracle (CPU only).

"KV Cache Mechanism Explained", section 8, item 2 keeps a fixed-size cache window: once the
cache holds more than WINDOW_SIZE entries, only the last WINDOW_SIZE are kept. The page prints
the trimming step and no numbers, so the window oracle is pinned by two independent
formulations agreeing (the page's trim-after-append procedure against the slicing formula), by
closed forms (a window of one returns the newest value; a window at least the length changes
nothing), by invariance to everything before the window, by a Decimal evaluation of the worked
example of "LLM Inference Acceleration -- KV Cache", section 2.1 under a window of two, and by
block counts of the paged form.
"""
import json
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle.attention import (cached_decode, rolling_cached_decode, window_decode,
                              window_start)
from oracle.caches import PagedCache
from oracle.pool import E_INVALID, PoolError, PoolModel

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def test_window_start_closed_form():
    assert window_start(10, 0) == 0
    assert window_start(10, 3) == 7
    assert window_start(3, 10) == 0
    assert window_start(10, 10) == 0
    assert window_start(0, 4) == 0
    with pytest.raises(ValueError):
        window_start(5, -1)


@pytest.mark.parametrize("W", [1, 2, 5, 16, 17, 40])
def test_trim_procedure_equals_window_formula(W):
    """The page's procedure (append, trim to the last W, attend) and the formula (attend
    positions max(0, L-W) .. L-1 of the untrimmed cache) are written independently."""
    rng = np.random.default_rng(W)
    T, D = 45, 8
    Q, K, V = (rng.standard_normal((T, D)) for _ in range(3))
    steps = rolling_cached_decode(Q, K, V, 0.3, W)
    for t in range(T):
        np.testing.assert_allclose(steps[t], window_decode(Q[t], K[:t + 1], V[:t + 1], 0.3, W),
                                   rtol=0, atol=1e-15)


def test_window_of_one_returns_the_newest_value():
    rng = np.random.default_rng(3)
    T, D = 12, 4
    Q, K, V = (rng.standard_normal((T, D)) for _ in range(3))
    np.testing.assert_array_equal(rolling_cached_decode(Q, K, V, 0.5, 1), V)


def test_window_at_least_the_length_is_no_window():
    rng = np.random.default_rng(4)
    T, D = 20, 8
    Q, K, V = (rng.standard_normal((T, D)) for _ in range(3))
    full = cached_decode(Q, K, V, 0.25)
    np.testing.assert_array_equal(rolling_cached_decode(Q, K, V, 0.25, T), full)
    np.testing.assert_array_equal(rolling_cached_decode(Q, K, V, 0.25, 0), full)


def test_positions_before_the_window_have_no_influence():
    rng = np.random.default_rng(5)
    L, D, W = 50, 16, 13
    q, K, V = rng.standard_normal(D), rng.standard_normal((L, D)), rng.standard_normal((L, D))
    a = window_decode(q, K, V, 0.25, W)
    K2, V2 = K.copy(), V.copy()
    K2[:L - W] = rng.standard_normal((L - W, D)) * 100.0
    V2[:L - W] = np.nan
    np.testing.assert_array_equal(window_decode(q, K2, V2, 0.25, W), a)
    # the oldest position inside the window does count
    K3 = K.copy()
    K3[L - W] *= 3.0
    assert np.abs(window_decode(q, K3, V, 0.25, W) - a).max() > 1e-6


def _decimal_row(q, K, V, scale):
    """softmax(scale q.K^T).V in 50-digit Decimal arithmetic, written as loops."""
    getcontext().prec = 50
    d = lambda x: Decimal(repr(float(x)))
    s = [sum(d(q[i]) * d(k[i]) for i in range(len(q))) * d(scale) for k in K]
    m = max(s)
    e = [(x - m).exp() for x in s]
    z = sum(e)
    return [float(sum(e[j] * d(V[j][i]) for j in range(len(K))) / z) for i in range(len(q))]


def test_worked_example_under_a_window_of_two():
    """The third token of the worked example with a window of two attends tokens 2 and 3 only:
    a logistic mix of their value rows, checked against a Decimal evaluation."""
    with open(GOLD) as f:
        g = json.load(f)
    X = np.array(g["X_step2"])
    Q, K, V = X @ np.array(g["W_Q"]), X @ np.array(g["W_K"]), X @ np.array(g["W_V"])
    got = rolling_cached_decode(Q, K, V, g["scale"], 2)
    np.testing.assert_allclose(got[2], _decimal_row(Q[2], K[1:], V[1:], g["scale"]), rtol=0,
                               atol=1e-15)
    s1, s2 = g["scale"] * Q[2] @ K[1], g["scale"] * Q[2] @ K[2]
    w = 1.0 / (1.0 + np.exp(-(s2 - s1)))
    np.testing.assert_allclose(got[2], V[1] + w * (V[2] - V[1]), rtol=0, atol=1e-15)
    # the first two steps are unaffected by a window of two
    np.testing.assert_array_equal(got[:2], cached_decode(Q[:2], K[:2], V[:2], g["scale"]))


# ---- paged form ------------------------------------------------------------------------
def _held(pool, s):
    return sum(1 for b in pool.seqs[s]["table"] if b >= 0)


@pytest.mark.parametrize("W", [1, 15, 16, 17, 40, 64])
def test_slide_keeps_exactly_the_blocks_covering_the_window(W):
    """After each one-token step and a slide, a sequence of length L holds the blocks of
    positions max(0, L-W) .. L-1: (L-1)//16 - max(0, L-W)//16 + 1 of them, never more than
    ceil((W-1)/16) + 1 (brute force over L), and freed blocks return to the pool."""
    pool = PoolModel(64, 16, 64)
    s = pool.alloc()
    bound = -(-(W - 1) // 16) + 1
    peak = 0
    for L in range(1, 400):
        pool.append([s], 1)
        pool.slide([s], W)
        want = (L - 1) // 16 - max(0, L - W) // 16 + 1
        assert _held(pool, s) == want, L
        peak = max(peak, want)
        pool.check()
        assert pool.stats()["used"] == want
    assert peak == bound


def test_slide_returns_dropped_count_and_frees_by_first_fit():
    pool = PoolModel(8, 16, 8)
    s = pool.alloc()
    pool.append([s], 40)                      # blocks 0, 1, 2 (positions 0..39)
    assert pool.slide([s], 20) == 1           # window 20..39: block 0 (0..15) leaves
    assert pool.seqs[s]["table"] == [-1, 1, 2]
    assert pool.slide([s], 20) == 0           # nothing more to drop
    t = pool.alloc()
    pool.append([t], 1)
    assert pool.seqs[t]["table"] == [0]       # first fit reuses the freed block 0
    assert pool.slide([s], 0) == 0            # window 0: no window
    with pytest.raises(PoolError) as e:
        pool.slide([s], -1)
    assert e.value.code == E_INVALID


def test_slide_with_forks_releases_one_reference():
    """A shared prefix stays resident while another holder still references it."""
    pool = PoolModel(16, 16, 16)
    p = pool.alloc()
    pool.append([p], 48)                      # blocks 0, 1, 2
    c = pool.fork(p)
    pool.append([c], 20)                      # c: len 68, new blocks 3, 4
    pool.slide([c], 20)                       # c's window 48..67: drops 0, 1, 2 from c
    assert pool.seqs[c]["table"][:3] == [-1, -1, -1]
    assert [pool.refcount[b] for b in (0, 1, 2)] == [1, 1, 1]
    pool.check()
    pool.slide([p], 16)                       # p's window 32..47: drops 0, 1 from p
    assert [pool.refcount[b] for b in (0, 1, 2)] == [0, 0, 1]
    pool.check()
    f = pool.fork(c)                          # a fork of a slid sequence shares live blocks only
    assert pool.seqs[f]["table"] == pool.seqs[c]["table"]
    pool.check()
    pool.free(c)
    pool.free(f)
    pool.free(p)
    assert pool.stats()["used"] == 0


def test_paged_window_decode_equals_window_formula():
    """Decode through a slid pool's tables attends the window only (dropped blocks are never
    read) and equals the formula on the unpaged rows."""
    rng = np.random.default_rng(11)
    H, D, W = 2, 8, 23
    lens = [5, 23, 24, 70, 129]
    pool = PoolModel(64, 16, 16, order=rng.permutation(64))
    cache = PagedCache(64, H, D, "f32", fill=np.nan)
    seqs = [pool.alloc() for _ in lens]
    rows = {}
    for s, L in zip(seqs, lens):
        k = rng.standard_normal((L, H, D)).astype(np.float32)
        v = rng.standard_normal((L, H, D)).astype(np.float32)
        slots, _ = pool.append([s], L)
        cache.write(slots, k, v)
        rows[s] = (k, v)
    pool.slide(seqs, W)
    tables, tl = pool.block_table(seqs)
    q = rng.standard_normal((len(lens), H, D)).astype(np.float32)
    got = cache.decode(q, tables, tl, 0.3, window=W)
    for i, s in enumerate(seqs):
        k, v = rows[s]
        for h in range(H):
            np.testing.assert_allclose(got[i, h], window_decode(q[i, h], k[:, h], v[:, h], 0.3, W),
                                       rtol=0, atol=1e-15)
    with pytest.raises(ValueError):
        cache.decode(q, tables, tl, 0.3)      # without the window it would read a dropped block
