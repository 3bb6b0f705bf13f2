"""Calls at the batch limit the library states: 4096 sequences in one decode or prefill call
(the per-sequence block prefix that both kernels scan lives in LDS), checked against the oracle,
and one sequence more refused with KVC_E_INVALID."""
import numpy as np
import pytest

import workloads
from oracle.caches import ContigCache, PagedCache
from oracle.pool import PoolModel
from tests.gpu_util import TOL, check, dev, kvc, note, scale_of, to_dev, torch

pytestmark = pytest.mark.gpu

B_MAX = 4096


def _contig(d, B, H, S, D, g):
    """Contiguous f16 caches of B sequences with every position 0 .. S-1 written (one bulk
    append), and the oracle's copy."""
    K = workloads.normal(g, (B, S, H, D), "f16")
    V = workloads.normal(g, (B, S, H, D), "f16")
    ref = ContigCache(B, H, S, D, "f16", fill=np.nan)
    kc = torch.full((B, H, S, D), float("nan"), dtype=torch.float16, device=d)
    vc = torch.full_like(kc, float("nan"))
    p = np.zeros(B, np.int32)
    kvc.append_contig(kc, vc, to_dev(p, d), to_dev(K, d), to_dev(V, d))
    ref.append(p, K, V)
    return kc, vc, ref


def test_contig_decode_at_the_batch_limit():
    d = dev()
    note("contig decode, 4096 sequences")
    g = workloads.rng(93)
    H, S, D = 2, 40, 64
    kc, vc, ref = _contig(d, B_MAX, H, S, D, g)
    lens = g.integers(0, S + 1, size=B_MAX).astype(np.int32)
    lens[:4] = [0, 1, 16, S]
    q = workloads.normal(g, (B_MAX, H, D), "f16")
    got = kvc.decode_attn_contig(to_dev(q, d), kc, vc, to_dev(lens, d), S, scale=scale_of(D))
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), ref.decode(q, lens, scale_of(D)), TOL["f16"])
    one_more = torch.zeros((B_MAX + 1, H, 1, D), dtype=torch.float16, device=d)
    with pytest.raises(kvc.KvcError):
        kvc.decode_attn_contig(torch.zeros((B_MAX + 1, H, D), dtype=torch.float16, device=d),
                               one_more, one_more.clone(),
                               torch.ones(B_MAX + 1, dtype=torch.int32, device=d), 1)


def test_paged_decode_at_the_batch_limit():
    d = dev()
    note("paged decode, 4096 sequences")
    g = workloads.rng(94)
    H, D = 2, 128
    lens = g.integers(0, 41, size=B_MAX).astype(np.int32)
    lens[:3] = [0, 1, 16]
    N = int(sum(workloads.blocks_for(int(L)) for L in lens)) + 8
    MB = 3
    order = workloads.permutation(g, N)
    pool = kvc.Pool(N, MB, order=order)
    model = PoolModel(N, 16, MB, order=order)
    seqs = [pool.alloc() for _ in range(B_MAX)]
    for _ in range(B_MAX):
        model.alloc()
    parts = []
    for s, L in zip(seqs, lens):
        if L:
            slots, src, _ = pool.append([s], int(L))
            mslots, _ = model.append([s], int(L))
            assert list(slots) == mslots and len(src) == 0
            parts.append(slots)
    slots = np.concatenate(parts).astype(np.int64)
    k = workloads.normal(g, (len(slots), H, D), "f16")
    v = workloads.normal(g, (len(slots), H, D), "f16")
    ref = PagedCache(N, H, D, "f16", fill=np.nan)
    ref.write(slots, k, v)
    layer = kvc.PagedLayer.empty(N, H, D, "f16", device=d, fill=float("nan"))
    kvc.write_paged(layer, to_dev(slots, d), to_dev(k, d), to_dev(v, d))
    tables, tl = pool.block_table(seqs)
    q = workloads.normal(g, (B_MAX, H, D), "f16")
    got = kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d),
                                int(lens.max()), scale=scale_of(D))
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), ref.decode(q, tables, tl, scale_of(D)), TOL["f16"])
    t1 = np.concatenate([tables, tables[:1]])
    l1 = np.concatenate([tl, tl[:1]])
    with pytest.raises(kvc.KvcError):
        kvc.decode_attn_paged(torch.zeros((B_MAX + 1, H, D), dtype=torch.float16, device=d),
                              layer, to_dev(t1, d), to_dev(l1, d), int(lens.max()))


def test_contig_prefill_at_the_batch_limit():
    """4096 sequences, each with a chunk of 0 to 3 new tokens at the end of its length."""
    d = dev()
    note("contig prefill, 4096 sequences")
    g = workloads.rng(95)
    H, G, S, D = 1, 2, 40, 64
    kc, vc, ref = _contig(d, B_MAX, H, S, D, g)
    lens = g.integers(1, S + 1, size=B_MAX).astype(np.int32)
    chunk = np.minimum(lens, g.integers(0, 4, size=B_MAX)).astype(np.int32)
    chunk[:2] = [0, 3]
    qs = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = workloads.normal(g, (int(qs[-1]), H * G, D), "f16")
    got = kvc.prefill_contig(to_dev(q, d), kc, vc, to_dev(qs, d), to_dev(lens, d),
                             scale=scale_of(D))
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), ref.prefill(q, qs, lens, scale_of(D)), TOL["f16"])
    one_more = torch.zeros((B_MAX + 1, H, 1, D), dtype=torch.float16, device=d)
    qs1 = np.ones(B_MAX + 2, np.int32)   # one token for the first sequence, none for the rest
    qs1[0] = 0
    with pytest.raises(kvc.KvcError):
        kvc.prefill_contig(torch.zeros((1, H * G, D), dtype=torch.float16, device=d), one_more,
                           one_more.clone(), to_dev(qs1, d),
                           torch.ones(B_MAX + 1, dtype=torch.int32, device=d))
