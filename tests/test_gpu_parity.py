"""HIP path vs the CPU oracle at small sizes (several tiles, ragged tails, edge cases).

Every kernel instantiation is exercised: contiguous f32/f16 x D 64/128, paged f32/f16/e4m3 x D
64/128, the append/scatter/copy kernels, and the fp8 writer. Cache contents are compared bit for
bit; attention outputs within max-abs 1e-5 (f32 cache), 2e-3 (f16), 3e-2 (e4m3) of the fp64
oracle. Unused cache slots hold NaN so any read past a sequence's length shows up.
"""
import numpy as np
import pytest

import workloads
from oracle.attention import cached_decode, decode_row
from oracle.caches import ContigCache, PagedCache
from oracle.codecs import e4m3_decode_table
from oracle.pool import PoolModel
from tests.gpu_util import TD, TOL, check, dev, kvc, max_err, note, scale_of, to_dev, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("f16", 64), ("f16", 128)])
@pytest.mark.parametrize("out_dtype", ["same", "f32"])
def test_contig_ragged(dtype, D, out_dtype):
    d = dev()
    note(f"contig ragged {dtype} D={D} out={out_dtype}")
    g = workloads.rng(100 + D)
    lens = [0, 1, 15, 16, 17, 33, 300]
    B, H, S = len(lens), 3, 320
    K = workloads.normal(g, (B, S, H, D), dtype)
    V = workloads.normal(g, (B, S, H, D), dtype)
    q = workloads.normal(g, (B, H, D), dtype)
    ref = ContigCache(B, H, S, D, dtype, fill=np.nan)
    kc = torch.full((B, H, S, D), float("nan"), dtype=TD[dtype], device=d)
    vc = torch.full_like(kc, float("nan"))
    pos = np.zeros(B, dtype=np.int32)
    n = max(lens)
    # bulk prefill of each sequence up to its length (positions >= length stay NaN)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        p = np.zeros(B, dtype=np.int32)
        p[:] = S  # other sequences: out of range, skipped
        p[b] = 0
        kvc.append_contig(kc, vc, to_dev(p, d), to_dev(K[:, :L], d), to_dev(V[:, :L], d))
        ref.append(p, K[:, :L], V[:, :L])
    np.testing.assert_array_equal(kc.cpu().numpy(), ref.K)   # NaN-aware, bitwise for numbers
    np.testing.assert_array_equal(vc.cpu().numpy(), ref.V)
    out = None if out_dtype == "same" else torch.empty((B, H, D), dtype=torch.float32, device=d)
    got = kvc.decode_attn_contig(to_dev(q, d), kc, vc, to_dev(np.array(lens, np.int32), d), n,
                                 scale=scale_of(D), out=out)
    torch.cuda.synchronize()
    want = ref.decode(q, lens, scale_of(D))
    tol = TOL[dtype] if (out_dtype == "f32" or dtype == "f32") else TOL["f16"]
    check(got.float().cpu().numpy(), want, tol)
    assert (got[0].float().abs().sum().item()) == 0.0    # L = 0 gives a zero row


def test_tiny_gpt_decode_every_step():
    """Tiny char-GPT shape, fp32, contiguous: 16-token prefill then 240 decode steps (append
    then attend); every step's output against the naive cached loop of the oracle."""
    d = dev()
    w = workloads.TINY_GPT
    note("tiny gpt 240 steps")
    g = workloads.rng(w.seed)
    T, H, D = w.ctx, w.heads, w.head_dim
    Q = workloads.normal(g, (1, T, H, D), "f32")
    K = workloads.normal(g, (1, T, H, D), "f32")
    V = workloads.normal(g, (1, T, H, D), "f32")
    kc = torch.full((1, H, w.s_max, D), float("nan"), device=d)
    vc = torch.full_like(kc, float("nan"))
    P = w.extra["prefill"]
    kvc.append_contig(kc, vc, to_dev(np.zeros(1, np.int32), d), to_dev(K[:, :P], d),
                      to_dev(V[:, :P], d))
    ws = kvc.new_workspace(1, H, D, device=d)
    outs = []
    lens_d = torch.zeros(1, dtype=torch.int32, device=d)
    for t in range(P, T):
        lens_d.fill_(t + 1)
        kvc.append_contig(kc, vc, to_dev(np.array([t], np.int32), d), to_dev(K[:, t:t + 1], d),
                          to_dev(V[:, t:t + 1], d))
        outs.append(kvc.decode_attn_contig(to_dev(Q[:, t], d), kc, vc, lens_d, t + 1,
                                           scale=w.scale, workspace=ws))
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=1).cpu().numpy()[0]           # [steps, H, D]
    for h in range(H):
        want = cached_decode(Q[0, P:, h], K[0, P:, h], V[0, P:, h], w.scale,
                             prefix_K=K[0, :P, h], prefix_V=V[0, :P, h])
        check(got[:, h], want, TOL["f32"])
    np.testing.assert_array_equal(kc.cpu().numpy()[0], K[0].transpose(1, 0, 2))


def _paged_setup(d, dtype, D, lens, H=3, seed=0, extra_blocks=5, new_dtype=None):
    """Pool + device layer + oracle cache holding sequences of the given lengths, written through
    kvc_write_paged in per-sequence bulk appends."""
    g = workloads.rng(seed)
    N = sum(workloads.blocks_for(L) for L in lens) + extra_blocks
    MB = max(workloads.blocks_for(L) for L in lens) + 2
    order = workloads.permutation(g, N)
    pool = kvc.Pool(N, MB, order=order)
    model = PoolModel(N, 16, MB, order=order)
    seqs = [pool.alloc() for _ in lens]
    for _ in lens:
        model.alloc()
    layer = kvc.PagedLayer.empty(N, H, D, dtype, device=d, fill=float("nan"))
    ref = PagedCache(N, H, D, dtype, fill=np.nan)
    src_dtype = new_dtype or ("f16" if dtype in ("e4m3", "i8") else dtype)
    data = []
    for s, L in zip(seqs, lens):
        slots, src, _ = pool.append([s], L)
        mslots, _ = model.append([s], L)
        assert list(slots) == mslots and len(src) == 0
        k = workloads.normal(g, (L, H, D), src_dtype)
        v = workloads.normal(g, (L, H, D), src_dtype)
        data.append((k, v))
        ref.write(slots, k, v)
        if L:
            kvc.write_paged(layer, to_dev(slots, d), to_dev(k, d), to_dev(v, d))
    return g, pool, model, seqs, layer, ref, data


def _compare_pools(layer, ref):
    torch.cuda.synchronize()
    np.testing.assert_array_equal(layer.k_pool.cpu().numpy(), ref.K)
    np.testing.assert_array_equal(layer.v_pool.cpu().numpy(), ref.V)
    if ref.k_scale is not None:
        np.testing.assert_array_equal(layer.k_scale.cpu().numpy(), ref.k_scale)
        np.testing.assert_array_equal(layer.v_scale.cpu().numpy(), ref.v_scale)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("f16", 64), ("f16", 128),
                                     ("e4m3", 64), ("e4m3", 128), ("i8", 64), ("i8", 128)])
def test_paged_ragged(dtype, D):
    d = dev()
    note(f"paged ragged {dtype} D={D}")
    lens = [1, 15, 16, 17, 250, 513, 0, 64]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, lens, seed=D)
    _compare_pools(layer, ref)
    tables, tl = pool.block_table(seqs)
    qdt = "f32" if dtype == "f32" else "f16"
    q = workloads.normal(g, (len(lens), 3, D), qdt)
    got = kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d), max(lens),
                                scale=scale_of(D))
    torch.cuda.synchronize()
    want = ref.decode(q, tables, tl, scale_of(D))
    check(got.float().cpu().numpy(), want, TOL["f32"] if dtype == "f32" else TOL["f16"])
    if dtype in ("e4m3", "i8"):
        # against the unquantised inputs as well, where enough positions are averaged: one
        # position alone reproduces a single dequantised row (e4m3 steps are 2^-4 relative)
        raw = PagedCache(layer.num_blocks, 3, D, "f32")
        for s, (k, v) in zip(seqs, data):
            t, L = pool.block_table([s])
            slots = [t[0][i // 16] * 16 + i % 16 for i in range(L[0])]
            raw.write(slots, k.astype(np.float32), v.astype(np.float32))
        long_ = [i for i, L in enumerate(lens) if L >= 250]
        unq = raw.decode(q, tables, tl, scale_of(D))
        check(got.float().cpu().numpy()[long_], unq[long_], TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_paged_equals_contiguous_on_gpu(dtype):
    d = dev()
    note(f"paged vs contiguous {dtype}")
    lens = [5, 16, 31, 200]
    D, H = 128, 3
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, lens, H=H, seed=9)
    S = 208
    kc = torch.zeros((len(lens), H, S, D), dtype=TD[dtype], device=d)
    vc = torch.zeros_like(kc)
    for b, (k, v) in enumerate(data):
        kc[b, :, :lens[b]] = to_dev(k.transpose(1, 0, 2), d)
        vc[b, :, :lens[b]] = to_dev(v.transpose(1, 0, 2), d)
    tables, tl = pool.block_table(seqs)
    q = to_dev(workloads.normal(g, (len(lens), H, D), dtype), d)
    out_f32 = torch.empty(q.shape, dtype=torch.float32, device=d)
    a = kvc.decode_attn_paged(q, layer, to_dev(tables, d), to_dev(tl, d), 200, out=out_f32)
    b = kvc.decode_attn_contig(q, kc, vc, to_dev(tl, d), 200,
                               out=torch.empty_like(out_f32)).cpu().numpy()
    check(a.cpu().numpy(), b, 1e-6)


def test_e4m3_hardware_decode_matches_definition_for_every_code():
    """L = 1, all-zero keys and V scale 1: the output row is exactly the decoded V codes."""
    d = dev()
    note("e4m3 code table through attention")
    D, H = 128, 1
    layer = kvc.PagedLayer.empty(2, H, D, "e4m3", device=d)
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    layer.v_pool[0, 0, 0] = to_dev(codes[:128], d)
    layer.v_pool[1, 0, 0] = to_dev(codes[128:], d)
    layer.k_scale.fill_(1.0)
    layer.v_scale.fill_(1.0)
    tables = to_dev(np.array([[0], [1]], np.int32), d)
    lens = to_dev(np.array([1, 1], np.int32), d)
    q = torch.ones((2, H, D), dtype=torch.float16, device=d)
    out = torch.empty((2, H, D), dtype=torch.float32, device=d)
    kvc.decode_attn_paged(q, layer, tables, lens, 1, out=out)
    got = out.cpu().numpy().reshape(256)
    want = e4m3_decode_table()[codes]
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("G", [1, 4])
def test_i8_decode_matches_definition_for_every_code(G):
    """L = 1 and V scale 1: the output row is exactly the int8 V codes, all 256 of them, on the
    vector kernel (G = 1) and on the matrix cores (G = 4, codes through fp16)."""
    d = dev()
    note(f"int8 code table through attention G={G}")
    D, H = 128, 1
    layer = kvc.PagedLayer.empty(2, H, D, "i8", device=d)
    codes = np.arange(-128, 128, dtype=np.int8)
    layer.v_pool[0, 0, 0] = to_dev(codes[:128], d)
    layer.v_pool[1, 0, 0] = to_dev(codes[128:], d)
    layer.k_scale.fill_(1.0)
    layer.v_scale.fill_(1.0)
    tables = to_dev(np.array([[0], [1]], np.int32), d)
    lens = to_dev(np.array([1, 1], np.int32), d)
    q = torch.ones((2, H * G, D), dtype=torch.float16, device=d)
    out = torch.empty((2, H * G, D), dtype=torch.float32, device=d)
    kvc.decode_gqa_paged(q, layer, tables, lens, 1, out=out)
    got = out.cpu().numpy()
    for r in range(G):
        np.testing.assert_array_equal(got[:, r].reshape(256), codes.astype(np.float64))


@pytest.mark.parametrize("fmt", ["e4m3", "i8"])
@pytest.mark.parametrize("src", ["f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_q8_writes_bit_exact_with_requantisation_and_block_reuse(fmt, src, D):
    """Token-by-token appends of growing magnitude force scale growth and requantisation; a freed
    block is reused (stale scale must be ignored at slot 0). e4m3 and int8 pools."""
    d = dev()
    note(f"8-bit writes {fmt} src={src} D={D}")
    H, N, MB = 5, 12, 6
    g = workloads.rng(77 + D)
    pool = kvc.Pool(N, MB)
    model = PoolModel(N, 16, MB)
    layer = kvc.PagedLayer.empty(N, H, D, fmt, device=d)
    ref = PagedCache(N, H, D, fmt)
    a, b = pool.alloc(), pool.alloc()
    model.alloc(), model.alloc()

    def append(seqs, n, mag):
        slots, src_, dst_ = pool.append(seqs, n)
        ms, cow = model.append(seqs, n)
        assert list(slots) == ms and list(zip(src_.tolist(), dst_.tolist())) == cow
        k = (workloads.normal(g, (len(slots), H, D), "f32") * mag).astype(np.float32)
        v = (workloads.normal(g, (len(slots), H, D), "f32") * mag * 0.5).astype(np.float32)
        if src == "f16":
            k, v = k.astype(np.float16), v.astype(np.float16)
        if len(cow):
            kvc.copy_blocks(layer, to_dev(src_, d), to_dev(dst_, d))
            ref.copy_blocks(cow)
        kvc.write_paged(layer, to_dev(slots, d), to_dev(k, d), to_dev(v, d))
        ref.write(slots, k, v)

    append([a], 20, 1.0)                      # bulk: one full block and 4 tokens
    for i in range(14):                       # single tokens of growing magnitude
        append([a, b], 1, 1.0 + 0.4 * i)
    c = pool.fork(a)
    model.fork(a)
    append([c, a], 3, 7.0)                    # copy-on-write of a's partial block
    pool.free(b)
    model.free(b)
    append([c], 40, 0.25)                     # reuses b's blocks: slot 0 restarts the scale
    _compare_pools(layer, ref)
    seqs = [a, c]
    tables, tl = pool.block_table(seqs)
    q = workloads.normal(g, (2, H, D), "f16")
    out = torch.empty((2, H, D), dtype=torch.float32, device=d)   # inputs reach ~7x unit scale
    got = kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d), 100,
                                scale=scale_of(D), out=out)
    check(got.cpu().numpy(), ref.decode(q, tables, tl, scale_of(D)), 2e-3)


@pytest.mark.parametrize("dtype", ["f16", "e4m3", "i8"])
def test_parallel_sampling_small_copy_on_write(dtype):
    """A 20-token prompt (partial last block) shared by 4 candidates; each appends 30 tokens with
    attention at every step; pools and outputs against the oracle."""
    d = dev()
    note(f"small parallel sampling {dtype}")
    H, D, N, MB = 4, 128, 40, 4
    g = workloads.rng(5)
    pool = kvc.Pool(N, MB)
    model = PoolModel(N, 16, MB)
    layer = kvc.PagedLayer.empty(N, H, D, dtype, device=d, fill=float("nan"))
    ref = PagedCache(N, H, D, dtype, fill=np.nan)
    p = pool.alloc()
    model.alloc()
    slots, _, _ = pool.append([p], 20)
    model.append([p], 20)
    k = workloads.normal(g, (20, H, D), "f16")
    v = workloads.normal(g, (20, H, D), "f16")
    kvc.write_paged(layer, to_dev(slots, d), to_dev(k, d), to_dev(v, d))
    ref.write(slots, k, v)
    seqs = [p] + [pool.fork(p) for _ in range(3)]
    for _ in range(3):
        model.fork(p)
    ws = kvc.new_workspace(4, H, D, device=d)
    n_copies = 0
    for step in range(30):
        slots, src_, dst_ = pool.append(seqs, 1)
        ms, cow = model.append(seqs, 1)
        assert list(slots) == ms
        n_copies += len(cow)
        if len(cow):
            kvc.copy_blocks(layer, to_dev(src_, d), to_dev(dst_, d))
            ref.copy_blocks(cow)
        k = workloads.normal(g, (4, H, D), "f16")
        v = workloads.normal(g, (4, H, D), "f16")
        kvc.write_paged(layer, to_dev(slots, d), to_dev(k, d), to_dev(v, d))
        ref.write(slots, k, v)
        tables, tl = pool.block_table(seqs)
        q = workloads.normal(g, (4, H, D), "f16")
        got = kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d),
                                    int(tl.max()), scale=scale_of(D), workspace=ws)
        if step in (0, 11, 29):
            check(got.float().cpu().numpy(), ref.decode(q, tables, tl, scale_of(D)), 2e-3,
                  f"step {step}")
    assert n_copies == 3
    _compare_pools(layer, ref)


def test_edge_cases_clamped_lengths_bad_ids_and_empty_batch():
    d = dev()
    note("edge cases")
    D, H = 128, 2
    lens = [20, 40]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, lens, H=H, seed=3)
    tables, tl = pool.block_table(seqs)
    q = workloads.normal(g, (2, H, D), "f16")
    scale = scale_of(D)
    # a length beyond the table capacity is clamped to it; a negative length is 0
    cap = tables.shape[1] * 16
    big = np.array([10 ** 6, -5], np.int32)
    t2 = tables.copy()
    got = kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(t2, d), to_dev(big, d), 64)
    torch.cuda.synchronize()
    assert got[1].float().abs().sum().item() == 0.0
    # an out-of-range block id makes its block contribute nothing
    t3 = tables.copy()
    t3[1, 1] = 10 ** 7
    t3[0, 0] = -3
    got = kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(t3, d), to_dev(tl, d), 64, scale=scale)
    want = np.zeros((2, H, D))
    for b in range(2):
        K, V = ref.gather(tables[b], tl[b])
        keep = [t for t in range(tl[b]) if t3[b, t // 16] == tables[b, t // 16]]
        for h in range(H):
            want[b, h] = decode_row(q[b, h], K[h][keep], V[h][keep], scale)
    check(got.float().cpu().numpy(), want, 2e-3)
    # an underestimated max_ctx only changes the grid, not the result
    a = kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d), 1)
    b_ = kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d), 40)
    assert max_err(a.float().cpu().numpy(), b_.float().cpu().numpy()) == 0.0
    # B = 0 is a no-op
    kvc.decode_attn_paged(torch.empty((0, H, D), dtype=torch.float16, device=d), layer,
                          torch.empty((0, 4), dtype=torch.int32, device=d),
                          torch.empty(0, dtype=torch.int32, device=d), 0)
    # bad arguments are refused before any launch
    with pytest.raises(kvc.KvcError):
        kvc.decode_attn_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d), 64,
                              workspace=torch.empty(16, dtype=torch.uint8, device=d))


def test_two_phase_api_equals_single_call():
    d = dev()
    note("two-phase api")
    lens = [300, 7, 1000]
    D, H = 128, 4
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, lens, H=H, seed=4)
    tables, tl = pool.block_table(seqs)
    q = to_dev(workloads.normal(g, (3, H, D), "f16"), d)
    tdv, tlv = to_dev(tables, d), to_dev(tl, d)
    a = kvc.decode_attn_paged(q, layer, tdv, tlv, 1000)
    out, ws = kvc.decode_partial_paged(q, layer, tdv, tlv, 1000)
    kvc.decode_merge(3, H, D, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, out)


def test_workspace_reuse_across_shapes():
    """One workspace serves calls of different batch sizes in stream order, with results equal
    to those of a fresh workspace."""
    d = dev()
    note("workspace reuse")
    D, H = 128, 4
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, [300, 7, 1000, 64], H=H,
                                                          seed=4)
    tables, tl = pool.block_table(seqs)
    tdv, tlv = to_dev(tables, d), to_dev(tl, d)
    q = to_dev(workloads.normal(g, (4, H, D), "f16"), d)
    ws = kvc.new_workspace(4, H, D, device=d)
    ws.fill_(0xA5)   # arbitrary prior contents
    for rep in range(3):
        for B in (4, 2, 3):
            a = kvc.decode_attn_paged(q[:B].contiguous(), layer, tdv[:B].contiguous(),
                                      tlv[:B].contiguous(), 1000, workspace=ws)
            b_ = kvc.decode_attn_paged(q[:B].contiguous(), layer, tdv[:B].contiguous(),
                                       tlv[:B].contiguous(), 1000)
            torch.cuda.synchronize()
            assert torch.equal(a, b_), (rep, B)
