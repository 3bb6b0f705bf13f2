"""Rolling-window decode on the GPU vs the CPU oracle.

Sequence b attends its last `window` positions (the new token included). Paged pools are slid
with the same window first (dropped table entries are -1 and must never be read), and also
decoded unslid (positions before the window hold real data that must be masked). Ragged
lengths put the window's first position at every offset inside a block. Unused cache slots hold
NaN. A contiguous cache that holds only the window, as a ring of W slots, decodes through the
existing grouped entry point and must equal the page's trim-after-append procedure.
"""
import numpy as np
import pytest

import workloads
from oracle.attention import rolling_cached_decode
from oracle.caches import ContigCache
from tests.gpu_util import TD, TOL, check, dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _paged_setup

pytestmark = pytest.mark.gpu

LENS = [1, 15, 16, 17, 250, 513, 0, 64, 1000]


@pytest.mark.parametrize("dtype,D,H,G,W,slide", [
    ("f16", 128, 2, 1, 100, True), ("f16", 128, 2, 1, 17, False), ("f16", 64, 3, 1, 1, True),
    ("f32", 128, 2, 1, 16, True), ("f32", 64, 1, 1, 300, False),
    ("e4m3", 128, 2, 1, 33, True), ("e4m3", 64, 2, 1, 1000, True),
    ("f16", 128, 2, 4, 100, True), ("f16", 64, 2, 8, 47, False), ("f16", 128, 1, 16, 5, True),
    ("e4m3", 128, 2, 8, 250, True), ("f32", 128, 2, 2, 64, True),
    ("i8", 128, 2, 1, 100, True), ("i8", 128, 2, 8, 33, True)])
def test_paged_window_against_oracle(dtype, D, H, G, W, slide):
    d = dev()
    note(f"window paged {dtype} D={D} H_kv={H} G={G} W={W} slide={slide}")
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, LENS, H=H, seed=W + D + G)
    if slide:
        assert pool.slide(seqs, W) == model.slide(seqs, W)
        pool.check()
    tables, tl = pool.block_table(seqs)
    mt, _ = model.block_table(seqs)
    assert tables.tolist() == mt
    qdt = "f32" if dtype == "f32" else "f16"
    q = workloads.normal(g, (len(LENS), H * G, D), qdt)
    got = kvc.decode_window_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d), max(LENS),
                                  W, scale=scale_of(D))
    torch.cuda.synchronize()
    want = ref.decode(q, tables, tl, scale_of(D), window=W)
    check(got.float().cpu().numpy(), want, TOL["f32"] if dtype == "f32" else TOL["f16"],
          f"W={W}")
    assert got[LENS.index(0)].float().abs().sum().item() == 0.0


def test_window_covering_everything_equals_plain_decode_bit_for_bit():
    d = dev()
    note("window >= length vs plain decode")
    D, H = 128, 3
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, LENS, H=H, seed=5)
    tables, tl = pool.block_table(seqs)
    q = to_dev(workloads.normal(g, (len(LENS), H, D), "f16"), d)
    tdv, tlv = to_dev(tables, d), to_dev(tl, d)
    a = kvc.decode_window_paged(q, layer, tdv, tlv, max(LENS), max(LENS))
    b = kvc.decode_attn_paged(q, layer, tdv, tlv, max(LENS))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,D,G,W", [("f32", 64, 1, 40), ("f16", 128, 1, 100),
                                         ("f16", 128, 4, 17), ("f32", 128, 2, 1)])
def test_contig_window_against_oracle(dtype, D, G, W):
    d = dev()
    note(f"window contig {dtype} D={D} G={G} W={W}")
    H, S = 2, 1008
    B = len(LENS)
    gen = workloads.rng(400 + W)
    K = workloads.normal(gen, (B, S, H, D), dtype)
    V = workloads.normal(gen, (B, S, H, D), dtype)
    q = workloads.normal(gen, (B, H * G, D), dtype)
    ref = ContigCache(B, H, S, D, dtype, fill=np.nan)
    kc = torch.full((B, H, S, D), float("nan"), dtype=TD[dtype], device=d)
    vc = torch.full_like(kc, float("nan"))
    for b, L in enumerate(LENS):
        if L:
            p = np.full(B, S, np.int32)
            p[b] = 0
            kvc.append_contig(kc, vc, to_dev(p, d), to_dev(K[:, :L], d), to_dev(V[:, :L], d))
            ref.append(p, K[:, :L], V[:, :L])
    got = kvc.decode_window_contig(to_dev(q, d), kc, vc, to_dev(np.array(LENS, np.int32), d),
                                   max(LENS), W, scale=scale_of(D))
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), ref.decode(q, LENS, scale_of(D), window=W), TOL[dtype],
          f"W={W}")


def test_window_argument_errors():
    d = dev()
    note("window errors")
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", 64, [20], H=1, seed=1)
    tables, tl = pool.block_table(seqs)
    q = to_dev(workloads.normal(g, (1, 1, 64), "f16"), d)
    for w in (0, -3):
        with pytest.raises(kvc.KvcError):
            kvc.decode_window_paged(q, layer, to_dev(tables, d), to_dev(tl, d), 20, w)


def test_ring_cache_of_window_slots_matches_trim_procedure():
    """The tiny character-GPT shape (6 heads x 64, fp32) generating 150 tokens with a window of
    48: a contiguous ring of 48 slots (position p at slot p % 48) written by kvc_append_contig
    and decoded by kvc_decode_gqa_contig over min(L, 48) slots equals the page's procedure."""
    d = dev()
    note("ring cache")
    H, D, W, T = 6, 64, 48, 150
    gen = workloads.rng(9)
    Q = workloads.normal(gen, (T, H, D), "f32")
    K = workloads.normal(gen, (T, H, D), "f32")
    V = workloads.normal(gen, (T, H, D), "f32")
    kc = torch.full((1, H, W, D), float("nan"), dtype=torch.float32, device=d)
    vc = torch.full_like(kc, float("nan"))
    want = np.stack([rolling_cached_decode(Q[:, h], K[:, h], V[:, h], 0.125, W)
                     for h in range(H)], axis=1)                       # [T, H, D]
    outs = []
    for t in range(T):
        kvc.append_contig(kc, vc, to_dev(np.array([t % W], np.int32), d),
                          to_dev(K[t:t + 1][None], d), to_dev(V[t:t + 1][None], d))
        L = min(t + 1, W)
        outs.append(kvc.decode_gqa_contig(to_dev(Q[t][None], d), kc, vc,
                                          to_dev(np.array([L], np.int32), d), W, scale=0.125))
    torch.cuda.synchronize()
    got = torch.cat(outs).cpu().numpy()
    check(got, want, TOL["f32"], "ring")


def test_window_full_size():
    """LLaMA-13B shapes (B=32, H=40, D=128, fp16) at context 2048 with a window of 1024, slid
    pool, the benchmark's launch configuration: every (sequence, head) row against the oracle
    over the generated inputs."""
    from oracle.attention import window_decode
    d = dev()
    w = workloads.LLAMA13B_WINDOW
    B, H, D, W = w.batch, w.heads, w.head_dim, w.extra["window"]
    note("window full size")
    lens = np.full(B, w.ctx, dtype=np.int64)
    N = int(sum(workloads.blocks_for(L) for L in lens))
    MB = workloads.blocks_for(int(lens.max()))
    pool = kvc.Pool(N, MB, order=workloads.llama13b_pool_order(N, w.seed))
    seqs = [pool.alloc() for _ in range(B)]
    slots = np.concatenate([pool.append([s], int(L))[0] for s, L in zip(seqs, lens)])
    layer = kvc.PagedLayer.empty(N, H, D, "f16", device=d)
    k = workloads.torch_normal((len(slots), H, D), torch.float16, d, w.seed * 100 + 1)
    v = workloads.torch_normal((len(slots), H, D), torch.float16, d, w.seed * 100 + 2)
    kvc.write_paged(layer, torch.from_numpy(slots).to(d), k, v)
    pool.slide(seqs, W)
    tables, tl = pool.block_table(seqs)
    q = workloads.torch_normal((B, H, D), torch.float16, d, w.seed * 100 + 3)
    out = kvc.decode_window_paged(q, layer, torch.from_numpy(tables).to(d),
                                  torch.from_numpy(tl).to(d), int(tl.max()), W, scale=w.scale)
    torch.cuda.synchronize()
    kh, vh = k.float().cpu().numpy(), v.float().cpu().numpy()
    qh, oh = q.float().cpu().numpy(), out.float().cpu().numpy()
    base = np.concatenate([[0], np.cumsum(lens)])
    for b in range(B):
        rows = slice(int(base[b]), int(base[b + 1]))
        for h in range(H):
            check(oh[b, h], window_decode(qh[b, h], kh[rows, h], vh[rows, h], w.scale, W),
                  TOL["f16"], f"b={b} h={h}")
