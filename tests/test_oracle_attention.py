"""Pins for oracle.attention (CPU only).

The pages print the worked example's inputs but not its outputs, so the example is checked
against an independent 50-digit Decimal evaluation of the same computation, and the oracle's
paths are tied together by what the pages state: caching changes no result, earlier rows do not
change when a token is added, and the special cases with closed forms.
"""
import json
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

from oracle.attention import cached_decode, decode_row, full_causal

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _load():
    with open(GOLD) as f:
        return json.load(f)


def _dec_matmul(A, B):
    return [[sum(A[i][k] * B[k][j] for k in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def _decimal_attention(X, WQ, WK, WV, scale):
    """Masked attention of the worked example in 50-digit decimal arithmetic, written as loops."""
    getcontext().prec = 50
    D = lambda m: [[Decimal(repr(v)) for v in row] for row in m]
    X, WQ, WK, WV = D(X), D(WQ), D(WK), D(WV)
    s = Decimal(repr(scale))
    Q, K, V = _dec_matmul(X, WQ), _dec_matmul(X, WK), _dec_matmul(X, WV)
    T = len(X)
    rows = []
    for i in range(T):
        sc = [sum(Q[i][d] * K[j][d] for d in range(4)) * s for j in range(i + 1)]
        m = max(sc)
        e = [(x - m).exp() for x in sc]
        z = sum(e)
        rows.append([sum(e[j] * V[j][d] for j in range(i + 1)) / z for d in range(4)])
    return Q, K, V, rows


def _np(m):
    return np.array([[float(v) for v in r] for r in m])


def test_worked_example_matches_decimal_evaluation():
    g = _load()
    X = np.array(g["X_step2"])
    WQ, WK, WV = np.array(g["W_Q"]), np.array(g["W_K"]), np.array(g["W_V"])
    Q, K, V = X @ WQ, X @ WK, X @ WV
    out = full_causal(Q, K, V, g["scale"])
    _, _, _, rows = _decimal_attention(g["X_step2"], g["W_Q"], g["W_K"], g["W_V"], g["scale"])
    np.testing.assert_allclose(out, _np(rows), rtol=0, atol=1e-15)


def test_worked_example_cached_step_equals_last_recompute_row():
    """Caching K and V gives the same output as recomputing everything (section 2.2)."""
    g = _load()
    X = np.array(g["X_step2"])
    WQ, WK, WV = np.array(g["W_Q"]), np.array(g["W_K"]), np.array(g["W_V"])
    Q, K, V = X @ WQ, X @ WK, X @ WV
    full = full_causal(Q, K, V, g["scale"])
    # step 1: two prompt tokens cached; step 2: the third token's q over the grown cache
    cached = cached_decode(Q[2:], K[2:], V[2:], g["scale"], prefix_K=K[:2], prefix_V=V[:2])
    np.testing.assert_allclose(cached[0], full[2], rtol=0, atol=1e-15)
    # and against the Decimal value of the same row
    _, _, _, rows = _decimal_attention(g["X_step2"], g["W_Q"], g["W_K"], g["W_V"], g["scale"])
    np.testing.assert_allclose(cached[0], _np(rows)[2], rtol=0, atol=1e-15)


def test_worked_example_earlier_rows_unchanged_by_new_token():
    g = _load()
    WQ, WK, WV = np.array(g["W_Q"]), np.array(g["W_K"]), np.array(g["W_V"])
    X1, X2 = np.array(g["X_step1"]), np.array(g["X_step2"])
    r1 = full_causal(X1 @ WQ, X1 @ WK, X1 @ WV, g["scale"])
    r2 = full_causal(X2 @ WQ, X2 @ WK, X2 @ WV, g["scale"])
    np.testing.assert_array_equal(r1, r2[:2])


def test_first_row_is_v0_and_second_row_is_logistic_mix():
    """Closed forms: one position gives v0; two positions give v0 + sigmoid(s1 - s0) (v1 - v0)."""
    g = _load()
    X = np.array(g["X_step1"])
    Q, K, V = X @ np.array(g["W_Q"]), X @ np.array(g["W_K"]), X @ np.array(g["W_V"])
    out = full_causal(Q, K, V, g["scale"])
    np.testing.assert_array_equal(out[0], V[0])
    s0, s1 = g["scale"] * Q[1] @ K[0], g["scale"] * Q[1] @ K[1]
    w = 1.0 / (1.0 + np.exp(-(s1 - s0)))
    np.testing.assert_allclose(out[1], V[0] + w * (V[1] - V[0]), rtol=0, atol=1e-16)


def test_special_cases():
    rng = np.random.default_rng(7)
    L, D = 37, 16
    K, V = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    # q = 0: all scores equal -> arithmetic mean of V
    np.testing.assert_allclose(decode_row(np.zeros(D), K, V, 0.25), V.mean(axis=0), atol=1e-15)
    # constant V rows -> that row, whatever the scores
    c = rng.standard_normal(D)
    np.testing.assert_allclose(decode_row(rng.standard_normal(D), K, np.tile(c, (L, 1)), 0.3),
                               c, atol=1e-15)
    # one dominant score -> that position's value
    q = 50.0 * K[11] / np.linalg.norm(K[11])
    Kd = K.copy()
    Kd[11] = 10.0 * q
    np.testing.assert_allclose(decode_row(q, Kd, V, 1.0), V[11], atol=1e-12)
    # L = 0 -> zero vector, never NaN
    np.testing.assert_array_equal(decode_row(np.ones(D), np.zeros((0, D)), np.zeros((0, D)), 1.0),
                                  np.zeros(D))


def test_position_permutation_invariance_and_operand_roles():
    rng = np.random.default_rng(8)
    L, D = 29, 8
    q, K, V = rng.standard_normal(D), rng.standard_normal((L, D)), rng.standard_normal((L, D))
    perm = rng.permutation(L)
    a = decode_row(q, K, V, 0.35)
    np.testing.assert_allclose(decode_row(q, K[perm], V[perm], 0.35), a, atol=1e-14)
    # permuting K alone (mismatching keys and values) changes the result
    assert np.abs(decode_row(q, K[perm], V, 0.35) - a).max() > 1e-3
    # the scale multiplies the scores, so it is not the same as scaling V
    assert np.abs(decode_row(q, K, V, 0.7) - a).max() > 1e-3


@pytest.mark.parametrize("T,D,start", [(1, 4, 0), (17, 8, 0), (5, 64, 40)])
def test_cached_loop_equals_full_recompute(T, D, start):
    rng = np.random.default_rng(T * 100 + D)
    n = start + T
    Q, K, V = (rng.standard_normal((n, D)) for _ in range(3))
    full = full_causal(Q[start:], K, V, 0.125, start_pos=start)
    cached = cached_decode(Q[start:], K[start:], V[start:], 0.125,
                           prefix_K=K[:start], prefix_V=V[:start])
    np.testing.assert_allclose(cached, full, rtol=0, atol=1e-14)
    # full recompute over all n rows, then keep the last T: same rows
    np.testing.assert_allclose(full_causal(Q, K, V, 0.125)[start:], full, atol=1e-14)


# ---- shared key/value heads (MQA / GQA), "LLM Inference Acceleration -- KV Cache" section 6.2 ----
from oracle.attention import grouped_decode, kv_head_of  # noqa: E402


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (8, 1), (12, 4), (6, 3)])
def test_grouped_decode_equals_multi_head_on_repeated_kv_heads(Hq, Hkv):
    """Sharing a key/value head among G consecutive query heads is multi-head attention over a
    cache whose heads are each repeated G times in place; repeating the whole head list G
    times (a different grouping) must give a different answer unless G = 1 or Hkv = 1."""
    L, D, G = 37, 16, Hq // Hkv
    q, K, V = _rand((Hq, D), 1), _rand((Hkv, L, D), 2), _rand((Hkv, L, D), 3)
    got = grouped_decode(q, K, V, 0.25)
    Kr, Vr = np.repeat(K, G, axis=0), np.repeat(V, G, axis=0)
    want = np.stack([decode_row(q[h], Kr[h], Vr[h], 0.25) for h in range(Hq)])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    Kt, Vt = np.tile(K, (G, 1, 1)), np.tile(V, (G, 1, 1))
    other = np.stack([decode_row(q[h], Kt[h], Vt[h], 0.25) for h in range(Hq)])
    if G > 1 and Hkv > 1:
        assert np.abs(got - other).max() > 1e-3


def test_mqa_every_query_head_reads_the_one_shared_head():
    L, D, Hq = 50, 8, 5
    q, K, V = _rand((Hq, D), 4), _rand((1, L, D), 5), _rand((1, L, D), 6)
    got = grouped_decode(q, K, V, 0.5)
    for h in range(Hq):
        np.testing.assert_allclose(got[h], decode_row(q[h], K[0], V[0], 0.5), rtol=0, atol=0)
    same = grouped_decode(np.repeat(q[:1], Hq, axis=0), K, V, 0.5)
    assert (same == same[0]).all()


def test_grouped_decode_equal_keys_average_their_values():
    """Keys equal within each key/value head give uniform weights: every query head of a group
    gets the mean of that group's value rows (closed form)."""
    Hq, Hkv, L, D = 8, 2, 23, 4
    K = np.repeat(_rand((Hkv, 1, D), 7), L, axis=1)
    V = _rand((Hkv, L, D), 8)
    got = grouped_decode(_rand((Hq, D), 9), K, V, 1.0)
    for h in range(Hq):
        np.testing.assert_allclose(got[h], V[h // 4].mean(axis=0), rtol=0, atol=1e-14)


def test_kv_head_mapping_and_uneven_split():
    assert [kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [kv_head_of(h, 4, 4) for h in range(4)] == [0, 1, 2, 3]
    assert {kv_head_of(h, 7, 1) for h in range(7)} == {0}
    with pytest.raises(ValueError):
        kv_head_of(0, 6, 4)


def test_paged_and_contiguous_models_agree_with_shared_heads():
    from oracle.caches import ContigCache, PagedCache
    H, G, D, lens = 2, 3, 8, [5, 21, 0]
    B, S = len(lens), 32
    rng = np.random.default_rng(10)
    contig = ContigCache(B, H, S, D, "f32")
    paged = PagedCache(12, H, D, "f32")
    tables = np.full((B, 2), -1, np.int64)
    nxt = 11
    for b, L in enumerate(lens):
        k = rng.standard_normal((L, H, D)).astype(np.float32)
        v = rng.standard_normal((L, H, D)).astype(np.float32)
        pos = np.full(B, S, np.int32)
        pos[b] = 0
        kk = np.zeros((B, L, H, D), np.float32)
        vv = np.zeros((B, L, H, D), np.float32)
        kk[b], vv[b] = k, v
        contig.append(pos, kk, vv)
        slots = []
        for t in range(L):
            if t % 16 == 0:
                tables[b, t // 16] = nxt
                nxt -= 1
            slots.append(tables[b, t // 16] * 16 + t % 16)
        paged.write(slots, k, v)
    q = rng.standard_normal((B, H * G, D))
    np.testing.assert_allclose(paged.decode(q, tables, lens, 0.3), contig.decode(q, lens, 0.3),
                               rtol=0, atol=1e-14)
