"""Whole-block 8-bit compression (kvc_compress_blocks) on the GPU vs the CPU oracle.

Blocks of an fp16 or fp32 paged layer are re-encoded into an e4m3 or int8 layer with a fresh
per-block scale over their valid slots; the codes and scales must equal the oracle's bit for
bit (slots past a block's valid count hold NaN in the source and code 0 after). Sequences
compressed from an fp16 pool then decode from the 8-bit pool like the oracle's 8-bit model, and
keep growing there under the running-scale write rule.
"""
import numpy as np
import pytest

import workloads
from oracle.caches import PagedCache
from oracle.pool import PoolModel
from tests.gpu_util import TOL, check, dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _compare_pools, _paged_setup

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("src_dt,fmt,D,H", [
    ("f16", "i8", 128, 3), ("f16", "e4m3", 128, 3), ("f32", "i8", 64, 3), ("f32", "e4m3", 64, 3),
    ("f16", "i8", 64, 3),
    # fp16 blocks on the streaming kernel at 8 and 16 pieces per thread, on one 1024-thread
    # workgroup per unit (64 heads of 128), and too wide for either (two-pass kernel)
    ("f16", "i8", 128, 12), ("f16", "e4m3", 128, 32), ("f16", "i8", 128, 64),
    ("f16", "e4m3", 128, 64), ("f16", "i8", 128, 70), ("f16", "e4m3", 64, 140)])
def test_compress_blocks_against_oracle(src_dt, fmt, D, H):
    d = dev()
    note(f"compress blocks {src_dt} -> {fmt} D={D} H={H}")
    g = workloads.rng(700 + D + H)
    N, N8 = 24, 30
    src = PagedCache(N, H, D, src_dt, fill=np.nan)
    src.K[:] = workloads.normal(g, src.K.shape, src_dt)
    src.V[:] = workloads.normal(g, src.V.shape, src_dt)
    src.K[2, 1, 4, 7] = 37.5                      # one block with a large outlier
    pairs = []
    dst_ids = g.permutation(N8)[:N]
    n_valid = g.integers(0, 17, size=N)
    n_valid[:3] = [0, 16, 1]
    for i in range(N):
        n = int(n_valid[i])
        src.K[i, :, n:, :] = np.nan                # past the valid slots: never read
        src.V[i, :, n:, :] = np.nan
        pairs.append((i, int(dst_ids[i]), n))
    layer = kvc.PagedLayer(to_dev(src.K, d), to_dev(src.V, d))
    out = kvc.PagedLayer.empty(N8, H, D, fmt, device=d, fill=float("nan"))
    ref = PagedCache(N8, H, D, fmt, fill=np.nan)
    kvc.compress_blocks(layer, out, to_dev(np.arange(N, dtype=np.int32), d),
                        to_dev(dst_ids.astype(np.int32), d), to_dev(n_valid.astype(np.int32), d))
    ref.compress_from(src, pairs)
    _compare_pools(out, ref)


def test_compress_all_slots_when_no_counts_given():
    d = dev()
    note("compress blocks, n_valid null")
    g = workloads.rng(9)
    H, D, N = 2, 128, 5
    src = PagedCache(N, H, D, "f16")
    src.K[:] = workloads.normal(g, src.K.shape, "f16")
    src.V[:] = workloads.normal(g, src.V.shape, "f16")
    layer = kvc.PagedLayer(to_dev(src.K, d), to_dev(src.V, d))
    out = kvc.PagedLayer.empty(N, H, D, "i8", device=d)
    ref = PagedCache(N, H, D, "i8")
    ids = to_dev(np.arange(N, dtype=np.int32), d)
    kvc.compress_blocks(layer, out, ids, ids)
    ref.compress_from(src, [(i, i, 16) for i in range(N)])
    _compare_pools(out, ref)


@pytest.mark.parametrize("fmt", ["i8", "e4m3"])
def test_compressed_sequences_decode_and_keep_growing(fmt):
    """Sequences of an fp16 pool move to an 8-bit pool (same lengths, fresh block ids there),
    decode from it, then take 20 more tokens each under the running-scale rule."""
    d = dev()
    note(f"compress sequences -> {fmt}")
    D, H = 128, 2
    lens = [1, 15, 16, 17, 250, 64, 0, 33]
    g, pool, model, seqs, layer, ref16, data = _paged_setup(d, "f16", D, lens, H=H, seed=71)
    tables16, _ = pool.block_table(seqs)
    N8 = sum(workloads.blocks_for(L + 20) for L in lens) + 3
    MB8 = max(workloads.blocks_for(L + 20) for L in lens) + 1
    order = workloads.permutation(g, N8)
    pool8 = kvc.Pool(N8, MB8, order=order)
    model8 = PoolModel(N8, 16, MB8, order=order)
    seqs8 = [pool8.alloc() for _ in lens]
    for _ in lens:
        model8.alloc()
    for s8, L in zip(seqs8, lens):
        assert list(pool8.append([s8], L)[0]) == model8.append([s8], L)[0]
    tables8, tl8 = pool8.block_table(seqs8)
    pairs = []
    for b, L in enumerate(lens):
        for j in range(workloads.blocks_for(L)):
            pairs.append((int(tables16[b][j]), int(tables8[b][j]), min(16, L - 16 * j)))
    layer8 = kvc.PagedLayer.empty(N8, H, D, fmt, device=d, fill=float("nan"))
    ref8 = PagedCache(N8, H, D, fmt, fill=np.nan)
    p = np.array(pairs, dtype=np.int32)
    kvc.compress_blocks(layer, layer8, to_dev(p[:, 0], d), to_dev(p[:, 1], d), to_dev(p[:, 2], d))
    ref8.compress_from(ref16, pairs)
    _compare_pools(layer8, ref8)
    q = workloads.normal(g, (len(lens), H, D), "f16")
    got = kvc.decode_attn_paged(to_dev(q, d), layer8, to_dev(tables8, d), to_dev(tl8, d),
                                max(lens), scale=scale_of(D))
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), ref8.decode(q, tables8, tl8, scale_of(D)), TOL["f16"],
          "compressed decode")
    # against the uncompressed pool, a bound on the quantisation error (not parity): int8
    # steps are s/2 = max|x|/254, about 2e-2 at these N(0,1) values; an e4m3 value moves by up
    # to 2^-4 of itself, so outputs (|v| up to ~4) move by up to ~0.25
    bound = {"i8": 3e-2, "e4m3": 0.25}[fmt]
    check(got.float().cpu().numpy(), ref16.decode(q, tables16, [int(x) for x in lens],
                                                  scale_of(D)), bound, "vs fp16 pool")
    # keep growing in the 8-bit pool
    for s8 in seqs8:
        slots, src, _ = pool8.append([s8], 20)
        assert len(src) == 0
        k = workloads.normal(g, (20, H, D), "f16")
        v = workloads.normal(g, (20, H, D), "f16")
        kvc.write_paged(layer8, to_dev(slots, d), to_dev(k, d), to_dev(v, d))
        ref8.write(slots, k, v)
    _compare_pools(layer8, ref8)
    tables8, tl8 = pool8.block_table(seqs8)
    got = kvc.decode_attn_paged(to_dev(q, d), layer8, to_dev(tables8, d), to_dev(tl8, d),
                                int(tl8.max()), scale=scale_of(D))
    torch.cuda.synchronize()
    check(got.float().cpu().numpy(), ref8.decode(q, tables8, tl8, scale_of(D)), TOL["f16"],
          "after growth")


def test_compress_argument_errors():
    d = dev()
    note("compress errors")
    f16 = kvc.PagedLayer.empty(4, 2, 64, "f16", device=d)
    i8 = kvc.PagedLayer.empty(4, 2, 64, "i8", device=d)
    i8h = kvc.PagedLayer.empty(4, 3, 64, "i8", device=d)
    ids = to_dev(np.arange(2, dtype=np.int32), d)
    with pytest.raises(kvc.KvcError):
        kvc.compress_blocks(i8, f16, ids, ids)            # 8-bit source
    with pytest.raises(kvc.KvcError):
        kvc.compress_blocks(f16, f16, ids, ids)           # 16-bit destination
    with pytest.raises(kvc.KvcError):
        kvc.compress_blocks(f16, i8h, ids, ids)           # head counts differ
    with pytest.raises(ValueError):
        kvc.compress_blocks(f16, i8, ids, ids[:1])
    kvc.compress_blocks(f16, i8, ids[:0], ids[:0])        # nothing to do


def test_compress_skips_pairs_outside_the_pools():
    """A pair whose source or destination id lies outside its pool writes nothing; the other
    pairs of the call are compressed as usual."""
    d = dev()
    note("compress skips out-of-pool ids")
    g = workloads.rng(13)
    H, D, N = 2, 64, 4
    src = PagedCache(N, H, D, "f16")
    src.K[:] = workloads.normal(g, src.K.shape, "f16")
    src.V[:] = workloads.normal(g, src.V.shape, "f16")
    layer = kvc.PagedLayer(to_dev(src.K, d), to_dev(src.V, d))
    out = kvc.PagedLayer.empty(N, H, D, "i8", device=d, fill=float("nan"))
    ref = PagedCache(N, H, D, "i8", fill=np.nan)
    s_ids = np.array([0, -1, 2, N, 3], dtype=np.int32)
    d_ids = np.array([1, 0, N + 5, 2, -7], dtype=np.int32)
    kvc.compress_blocks(layer, out, to_dev(s_ids, d), to_dev(d_ids, d))
    ref.compress_from(src, [(0, 1, 16)])          # the only pair inside both pools
    _compare_pools(out, ref)


@pytest.mark.parametrize("fmt", ["i8", "e4m3"])
def test_compress_many_units_per_workgroup_with_skips(fmt):
    """3000 pairs (6000 units: each streaming workgroup walks about 23 of them) with every fifth
    pair outside a pool, so skipped units fall between encoded ones in each workgroup's walk:
    every encoded block against the oracle, bit for bit, and the skipped destinations untouched."""
    d = dev()
    note(f"compress many units with skips -> {fmt}")
    g = workloads.rng(14)
    H, D, N = 4, 64, 3000
    src = PagedCache(N, H, D, "f16")
    src.K[:] = workloads.normal(g, src.K.shape, "f16")
    src.V[:] = workloads.normal(g, src.V.shape, "f16")
    src.K[:, :, :, 3] *= g.uniform(0.01, 100.0, size=(N, 1, 1)).astype(np.float16)  # scales vary
    layer = kvc.PagedLayer(to_dev(src.K, d), to_dev(src.V, d))
    out = kvc.PagedLayer.empty(N, H, D, fmt, device=d, fill=float("nan"))
    ref = PagedCache(N, H, D, fmt, fill=np.nan)
    s_ids = g.permutation(N).astype(np.int32)
    d_ids = g.permutation(N).astype(np.int32)
    skip = np.arange(N) % 5 == 2
    s_ids[skip & (np.arange(N) % 2 == 0)] = N + 3       # source outside its pool
    d_ids[skip & (np.arange(N) % 2 == 1)] = -1          # destination outside its pool
    n_valid = g.integers(1, 17, size=N).astype(np.int32)
    kvc.compress_blocks(layer, out, to_dev(s_ids, d), to_dev(d_ids, d), to_dev(n_valid, d))
    ref.compress_from(src, [(int(s_ids[i]), int(d_ids[i]), int(n_valid[i]))
                            for i in range(N) if not skip[i]])
    _compare_pools(out, ref)


def _boundary_blocks(fmt, H, D, g):
    """Source blocks [N, H, 16, D] (fp16) whose quotients x/scale sit on or next to the format's
    rounding boundaries, plus degenerate maxima."""
    n = H * 16 * D
    blocks = []
    if fmt == "i8":
        # maximum 127 gives scale 1: every k + 1/2 is an exact tie between two codes
        ties = np.arange(-127, 127, dtype=np.float64) + 0.5
    else:
        # maximum 448 gives scale 1: midpoints of neighbouring e4m3 values are exact ties (four
        # significant bits, so exact in fp16), subnormal steps included
        from oracle.codecs import e4m3_decode
        vals = np.unique(np.abs(e4m3_decode(np.arange(0x7F, dtype=np.uint8))))
        ties = np.concatenate([(vals[1:] + vals[:-1]) / 2, vals])
    x = np.resize(ties, n) * np.where(g.random(n) < 0.5, -1.0, 1.0)
    x[0] = 127.0 if fmt == "i8" else 448.0
    blocks.append(x)
    blocks.append(np.where(g.random(n) < 0.5, -0.0, 0.0))          # all zeros: scale 0
    wide = g.standard_normal(n) * 10.0 ** g.uniform(-7, 0, n)       # many tiny quotients
    blocks.append(wide)
    blocks.append(g.standard_normal(n) * 1e-4)                      # fp16 subnormals
    if fmt == "i8":                                                 # non-finite maxima
        inf = g.standard_normal(n)
        inf[5] = np.inf
        blocks.append(inf)
        nan = g.standard_normal(n)
        nan[9] = np.nan
        blocks.append(nan)
    return np.stack([b.reshape(H, 16, D) for b in blocks]).astype(np.float16)


@pytest.mark.parametrize("fmt", ["i8", "e4m3"])
def test_compress_rounding_boundaries(fmt):
    """Ties, near-ties and degenerate block maxima at the long-context shape (32 heads of 128,
    the register-resident kernel): codes and scales equal the oracle's bit for bit."""
    d = dev()
    note(f"compress rounding boundaries -> {fmt}")
    H, D = 32, 128
    g = workloads.rng(33)
    blocks = _boundary_blocks(fmt, H, D, g)
    N = blocks.shape[0]
    src = PagedCache(N, H, D, "f16")
    src.K[:] = blocks
    src.V[:] = -blocks[::-1]
    layer = kvc.PagedLayer(to_dev(src.K, d), to_dev(src.V, d))
    out = kvc.PagedLayer.empty(N, H, D, fmt, device=d, fill=float("nan"))
    ref = PagedCache(N, H, D, fmt, fill=np.nan)
    ids = np.arange(N, dtype=np.int32)
    kvc.compress_blocks(layer, out, to_dev(ids, d), to_dev(ids[::-1].copy(), d))
    ref.compress_from(src, [(i, N - 1 - i, 16) for i in range(N)])
    _compare_pools(out, ref)


@pytest.mark.parametrize("fmt", ["i8", "e4m3"])
def test_compress_full_layer_sampled(fmt):
    """The benchmark's compression at full size (64 sequences x 4096 tokens, 32 heads x 128, one
    layer over a shuffled pool), in its launch configuration: every block compressed in one
    call; sampled blocks' codes and scales bit-exact against the oracle, which takes each
    block's values from the generated tensors through the slot map."""
    from oracle.codecs import compress_block
    d = dev()
    note(f"compress full layer -> {fmt}")
    w = workloads.COMPRESS_I8
    B, H, D, T = w.batch, w.heads, w.head_dim, w.ctx
    nblk = workloads.blocks_for(T)
    N = B * nblk
    pool = kvc.Pool(N, nblk, order=workloads.llama13b_pool_order(N, w.seed))
    seqs = [pool.alloc() for _ in range(B)]
    slots = np.concatenate([pool.append([s], T)[0] for s in seqs])
    src = kvc.PagedLayer.empty(N, H, D, "f16", device=d, fill=float("nan"))
    k = workloads.torch_normal((len(slots), H, D), torch.float16, d, 61)
    v = workloads.torch_normal((len(slots), H, D), torch.float16, d, 62)
    kvc.write_paged(src, torch.from_numpy(slots).to(d), k, v)
    tables, lens = pool.block_table(seqs)
    ids = np.concatenate([tables[b][:nblk] for b in range(B)]).astype(np.int32)
    nval = np.full(len(ids), 16, np.int32)
    dst = kvc.PagedLayer.empty(N, H, D, fmt, device=d, fill=float("nan"))
    ids_d = to_dev(ids, d)
    kvc.compress_blocks(src, dst, ids_d, ids_d, to_dev(nval, d))
    torch.cuda.synchronize()
    blk_of = slots // 16
    rng = np.random.default_rng(12)
    for p in rng.choice(ids, size=24, replace=False):
        tok = np.nonzero(blk_of == p)[0]
        assert len(tok) == 16
        order = np.argsort(slots[tok] % 16)
        tok_d = torch.from_numpy(tok[order]).to(d)
        for pool_g, sc_g, x in ((dst.k_pool, dst.k_scale, k), (dst.v_pool, dst.v_scale, v)):
            xb = x[tok_d].float().cpu().numpy().transpose(1, 0, 2)      # [H, 16, D]
            codes, s = compress_block(xb, 16, fmt)
            np.testing.assert_array_equal(pool_g[int(p)].cpu().numpy(), codes)
            assert sc_g[int(p)].item() == s
