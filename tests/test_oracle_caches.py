"""Pins for oracle.caches and oracle.accounting (CPU only)."""
import json
import os

import numpy as np

from oracle.accounting import (blocks_needed, kv_bytes, kv_bytes_per_token,
                               sampling_token_capacity, wasted_slots)
from oracle.attention import cached_decode, full_causal
from oracle.caches import ContigCache, PagedCache
from oracle.codecs import e4m3_decode, fp8_write_token
from oracle.pool import PoolModel

FIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_llama7b_bytes_per_token_and_context_sizes():
    assert kv_bytes_per_token(32, 32, 128, 2) == FIG["llama7b_kv_bytes_per_token"]["value"]
    for ctx, approx in FIG["llama7b_context_sizes_approx_bytes"]["value"].items():
        b = kv_bytes(32, 32, 128, int(ctx), 2)
        assert b == int(ctx) * 524288 and abs(b / approx - 1) < 0.08
    # one layer of LLaMA-7B at 1024 tokens is the 16 MB next to a 64-entry table
    assert kv_bytes(1, 32, 128, 1024, 2) == 16 * 2 ** 20


def test_llama13b_sequence_bytes():
    f = FIG["llama13b_seq_bytes_approx"]
    b = kv_bytes(40, 40, 128, 2048, 2)
    assert b == int(np.prod(f["factors"])) == 1_677_721_600
    assert abs(b / f["value"] - 1) < 0.05


def test_block_counts_and_sampling_capacity():
    assert blocks_needed(1024) == 64 and wasted_slots(1024) == 0
    assert max(wasted_slots(t) for t in range(1, 2000)) == 15
    f = FIG["parallel_sampling"]
    assert sampling_token_capacity(8, 1024, 128, shared=False) == f["capacity_unshared"]
    assert sampling_token_capacity(8, 1024, 128, shared=True) == f["capacity_shared"]


def test_contig_cache_matches_naive_cached_loop_and_recompute():
    rng = np.random.default_rng(21)
    B, H, S, D = 2, 3, 40, 16
    T = 33
    Q = rng.standard_normal((B, T, H, D)).astype(np.float32)
    K = rng.standard_normal((B, T, H, D)).astype(np.float32)
    V = rng.standard_normal((B, T, H, D)).astype(np.float32)
    c = ContigCache(B, H, S, D, "f32", fill=np.nan)
    prefill = 5
    c.append([0, 0], K[:, :prefill], V[:, :prefill])
    outs = []
    for t in range(prefill, T):
        c.append([t, t], K[:, t:t + 1], V[:, t:t + 1])
        outs.append(c.decode(Q[:, t], [t + 1, t + 1], 0.25))
    outs = np.stack(outs, axis=1)                     # [B, steps, H, D]
    for b in range(B):
        for h in range(H):
            ref = cached_decode(Q[b, prefill:, h], K[b, prefill:, h], V[b, prefill:, h], 0.25,
                                prefix_K=K[b, :prefill, h], prefix_V=V[b, :prefill, h])
            np.testing.assert_array_equal(outs[b, :, h], ref)
            full = full_causal(Q[b, :, h], K[b, :, h], V[b, :, h], 0.25)
            np.testing.assert_allclose(outs[b, :, h], full[prefill:], atol=1e-14)


def test_paged_equals_contiguous_bit_exact_through_shuffled_tables():
    rng = np.random.default_rng(22)
    H, D = 3, 16
    lens = [1, 16, 17, 45]
    B = len(lens)
    N = 20
    order = rng.permutation(N)
    pool = PoolModel(N, 16, 4, order=order)
    seqs = [pool.alloc() for _ in range(B)]
    pc = PagedCache(N, H, D, "f16", fill=np.nan)
    cc = ContigCache(B, H, 48, D, "f16", fill=np.nan)
    K = rng.standard_normal((B, 48, H, D)).astype(np.float16)
    V = rng.standard_normal((B, 48, H, D)).astype(np.float16)
    for b, s in enumerate(seqs):
        slots, cow = pool.append([s], lens[b])
        pc.write(slots, K[b, :lens[b]], V[b, :lens[b]])
    cc.append([0] * B, K, V)
    tables, got_lens = pool.block_table(seqs)
    assert got_lens == lens
    q = rng.standard_normal((B, H, D)).astype(np.float16)
    a = pc.decode(q, tables, lens, 0.25)
    b_ = cc.decode(q, lens, 0.25)
    np.testing.assert_array_equal(a, b_)
    assert np.isfinite(a).all()              # no NaN-filled unused slot was read


def test_paged_copy_on_write_keeps_shared_prefix_values():
    rng = np.random.default_rng(23)
    H, D = 2, 8
    pool = PoolModel(8, 16, 4)
    pc = PagedCache(8, H, D, "f32")
    a = pool.alloc()
    xk = rng.standard_normal((20, H, D)).astype(np.float32)
    xv = rng.standard_normal((20, H, D)).astype(np.float32)
    slots, _ = pool.append([a], 20)
    pc.write(slots, xk, xv)
    b = pool.fork(a)
    nk = rng.standard_normal((2, H, D)).astype(np.float32)
    slots, cow = pool.append([b, a], 1)
    pc.copy_blocks(cow)
    pc.write(slots, nk, nk)
    t, lens = pool.block_table([a, b])
    Ka, _ = pc.gather(t[0], lens[0])
    Kb, _ = pc.gather(t[1], lens[1])
    np.testing.assert_array_equal(Ka[:, :20], xk.transpose(1, 0, 2))
    np.testing.assert_array_equal(Kb[:, :20], xk.transpose(1, 0, 2))
    np.testing.assert_array_equal(Kb[:, 20], nk[0])
    np.testing.assert_array_equal(Ka[:, 20], nk[1])


def test_paged_fp8_write_is_token_sequential_and_decodes_codes_times_scale():
    rng = np.random.default_rng(24)
    H, D = 2, 8
    pc = PagedCache(3, H, D, "e4m3")
    x = rng.standard_normal((20, H, D)).astype(np.float16)
    slots = list(range(16, 32)) + [0, 1, 2, 3]
    pc.write(slots, x, x)
    codes = np.zeros((H, 16, D), dtype=np.uint8)
    s = np.float32(0)
    for t in range(16):
        s = fp8_write_token(codes, s, t, x[t])
    np.testing.assert_array_equal(pc.K[1], codes)
    assert pc.k_scale[1] == s and pc.v_scale[1] == s
    K, V = pc.gather([1, 0], 20)
    np.testing.assert_array_equal(K[:, :16], (e4m3_decode(codes) * np.float64(s)))



def test_paged_i8_write_is_token_sequential_and_decodes_codes_times_scale():
    from oracle.codecs import i8_decode, i8_write_token
    rng = np.random.default_rng(25)
    H, D = 2, 8
    pc = PagedCache(3, H, D, "i8", fill=np.nan)
    assert (pc.K == -128).all()              # unused slots hold the never-written code
    x = rng.standard_normal((20, H, D)).astype(np.float16)
    slots = list(range(16, 32)) + [0, 1, 2, 3]
    pc.write(slots, x, x)
    codes = np.zeros((H, 16, D), dtype=np.int8)
    s = np.float32(0)
    for t in range(16):
        s = i8_write_token(codes, s, t, x[t])
    np.testing.assert_array_equal(pc.K[1], codes)
    assert pc.k_scale[1] == s and pc.v_scale[1] == s
    K, V = pc.gather([1, 0], 20)
    np.testing.assert_array_equal(K[:, :16], i8_decode(codes) * np.float64(s))


# ---- chunked prefill through the cache models -----------------------------------------------
def test_prefill_rows_equal_decode_at_each_length_and_paged_equals_contig():
    """Row i of a prefill chunk is the decode of the same query at length start + i + 1 (the
    cached path reaches the recompute result, "LLM Inference Acceleration -- KV Cache", section
    2.2); the paged and contiguous models agree bit for bit; grouped heads read kv_head_of."""
    from oracle.pool import PoolModel
    rng = np.random.default_rng(21)
    H, G, D = 2, 2, 8
    lens = [1, 17, 40, 5]
    chunk = [1, 9, 40, 0]
    q_start = np.concatenate([[0], np.cumsum(chunk)])
    S = max(lens)
    contig = ContigCache(len(lens), H, S, D, "f32", fill=np.nan)
    pool = PoolModel(16, 16, 4, order=rng.permutation(16))
    paged = PagedCache(16, H, D, "f32", fill=np.nan)
    seqs = [pool.alloc() for _ in lens]
    for b, (s, L) in enumerate(zip(seqs, lens)):
        k = rng.standard_normal((1, L, H, D)).astype(np.float32)
        v = rng.standard_normal((1, L, H, D)).astype(np.float32)
        pos = np.full(len(lens), S, np.int32)
        pos[b] = 0
        kk = np.zeros((len(lens), L, H, D), np.float32)
        vv = np.zeros_like(kk)
        kk[b], vv[b] = k[0], v[0]
        contig.append(pos, kk, vv)
        slots, _ = pool.append([s], L)
        paged.write(slots, k[0], v[0])
    tables, tl = pool.block_table(seqs)
    q = rng.standard_normal((int(q_start[-1]), H * G, D)).astype(np.float32)
    a = contig.prefill(q, q_start, lens, 0.3)
    bp = paged.prefill(q, q_start, tables, tl, 0.3)
    np.testing.assert_array_equal(a, bp)
    for b, L in enumerate(lens):
        n = chunk[b]
        for i in range(n):
            row = int(q_start[b]) + i
            dec = contig.decode(q[row][None].repeat(len(lens), 0), [L - n + i + 1] * len(lens),
                                0.3)[b]
            np.testing.assert_allclose(a[row], dec, rtol=0, atol=1e-14)
