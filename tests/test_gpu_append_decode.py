"""Fused append + attend (one pass stores the new token's K/V and attends over the cache).

Against the separate write + decode calls of the same step: cache contents and outputs bit for
bit (the new row's values are the same and are visited in the same order). Against the oracle:
cache contents bit for bit, outputs within the tolerance of the cache dtype. Unused cache slots
hold NaN, so a row stored in the wrong place or read before it is written shows up.
"""
import numpy as np
import pytest

import workloads
from oracle.attention import cached_decode
from oracle.caches import ContigCache
from tests.gpu_util import TD, TOL, check, dev, kvc, note, scale_of, to_dev, torch
from tests.test_gpu_parity import _compare_pools, _paged_setup

pytestmark = pytest.mark.gpu

# lengths after the append: the new token opens a block (17, 33, 1), fills one (16, 64), or
# lands mid-block; 0 is an empty sequence that takes no token
LENS = [17, 1, 16, 250, 64, 0, 33, 513]


def _clone_layer(layer):
    return kvc.PagedLayer(layer.k_pool.clone(), layer.v_pool.clone())


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("f16", 64), ("f16", 128)])
def test_paged_fused_equals_write_then_decode(dtype, D):
    d = dev()
    note(f"append-decode paged {dtype} D={D}")
    H = 3
    prior = [max(L - 1, 0) for L in LENS]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, prior, H=H, seed=D + 1)
    live = [s for s, L in zip(seqs, LENS) if L > 0]
    slots, src, dst = pool.append(live, 1)
    ms, cow = model.append(live, 1)
    assert list(slots) == ms and not cow
    tables, tl = pool.block_table(seqs)
    assert list(tl) == LENS
    B = len(LENS)
    k_new = workloads.normal(g, (B, H, D), dtype)
    v_new = workloads.normal(g, (B, H, D), dtype)
    q = workloads.normal(g, (B, H, D), dtype)
    rows = [b for b, L in enumerate(LENS) if L > 0]
    ref.write(slots, k_new[rows], v_new[rows])
    tdv, tlv = to_dev(tables, d), to_dev(tl, d)
    qd, kd, vd = to_dev(q, d), to_dev(k_new, d), to_dev(v_new, d)
    other = _clone_layer(layer)
    fused = kvc.append_decode_paged(qd, layer, tdv, tlv, kd, vd, max(LENS), scale=scale_of(D))
    kvc.write_paged(other, to_dev(slots, d), to_dev(k_new[rows], d), to_dev(v_new[rows], d))
    plain = kvc.decode_attn_paged(qd, other, tdv, tlv, max(LENS), scale=scale_of(D))
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    assert torch.equal(layer.k_pool.view(torch.int8), other.k_pool.view(torch.int8))
    assert torch.equal(layer.v_pool.view(torch.int8), other.v_pool.view(torch.int8))
    _compare_pools(layer, ref)
    check(fused.float().cpu().numpy(), ref.decode(q, tables, tl, scale_of(D)), TOL[dtype])
    assert fused[LENS.index(0)].float().abs().sum().item() == 0.0


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f16", 128)])
def test_contig_fused_equals_append_then_decode(dtype, D):
    d = dev()
    note(f"append-decode contig {dtype} D={D}")
    H, S = 3, 528
    B = len(LENS)
    g = workloads.rng(200 + D)
    K = workloads.normal(g, (B, S, H, D), dtype)
    V = workloads.normal(g, (B, S, H, D), dtype)
    q = workloads.normal(g, (B, H, D), dtype)
    ref = ContigCache(B, H, S, D, dtype, fill=np.nan)
    kc = torch.full((B, H, S, D), float("nan"), dtype=TD[dtype], device=d)
    vc = torch.full_like(kc, float("nan"))
    for b, L in enumerate(LENS):           # prefill positions [0, L-1)
        if L > 1:
            p = np.full(B, S, np.int32)
            p[b] = 0
            kvc.append_contig(kc, vc, to_dev(p, d), to_dev(K[:, :L - 1], d),
                              to_dev(V[:, :L - 1], d))
            ref.append(p, K[:, :L - 1], V[:, :L - 1])
    pos = np.array([L - 1 if L > 0 else S for L in LENS], np.int32)
    k_new, v_new = K[np.arange(B), np.maximum(pos, 0) % S], V[np.arange(B), np.maximum(pos, 0) % S]
    ref.append(pos, k_new[:, None], v_new[:, None])
    kc2, vc2 = kc.clone(), vc.clone()
    lens = to_dev(np.array(LENS, np.int32), d)
    qd, kd, vd = to_dev(q, d), to_dev(k_new, d), to_dev(v_new, d)
    fused = kvc.append_decode_contig(qd, kc, vc, lens, kd, vd, max(LENS), scale=scale_of(D))
    kvc.append_contig(kc2, vc2, to_dev(pos, d), kd[:, None].contiguous(), vd[:, None].contiguous())
    plain = kvc.decode_attn_contig(qd, kc2, vc2, lens, max(LENS), scale=scale_of(D))
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    np.testing.assert_array_equal(kc.cpu().numpy(), ref.K)
    np.testing.assert_array_equal(vc.cpu().numpy(), ref.V)
    check(fused.float().cpu().numpy(), ref.decode(q, LENS, scale_of(D)), TOL[dtype])


def test_tiny_gpt_fused_every_step():
    """The fp32 tiny char-GPT shape decoded with the fused call at every step: outputs against
    the oracle's cached loop, final cache against the inputs."""
    d = dev()
    w = workloads.TINY_GPT
    note("append-decode tiny gpt 240 steps")
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
    Kd, Vd, Qd = to_dev(K, d), to_dev(V, d), to_dev(Q, d)
    lens_d = torch.zeros(1, dtype=torch.int32, device=d)
    outs = []
    for t in range(P, T):
        lens_d.fill_(t + 1)
        outs.append(kvc.append_decode_contig(Qd[:, t].contiguous(), kc, vc, lens_d,
                                             Kd[:, t].contiguous(), Vd[:, t].contiguous(), t + 1,
                                             scale=w.scale, workspace=ws))
    torch.cuda.synchronize()
    got = torch.stack(outs, dim=1).cpu().numpy()[0]
    for h in range(H):
        want = cached_decode(Q[0, P:, h], K[0, P:, h], V[0, P:, h], w.scale,
                             prefix_K=K[0, :P, h], prefix_V=V[0, :P, h])
        check(got[:, h], want, TOL["f32"])
    np.testing.assert_array_equal(kc.cpu().numpy()[0], K[0].transpose(1, 0, 2))
    np.testing.assert_array_equal(vc.cpu().numpy()[0], V[0].transpose(1, 0, 2))


def test_parallel_sampling_fused_with_copy_on_write():
    """A 20-token prompt shared by 4 candidates; 30 fused steps, the pool's copy-on-write pairs
    copied before each step's call."""
    from oracle.caches import PagedCache
    from oracle.pool import PoolModel
    d = dev()
    note("append-decode parallel sampling")
    H, D, N, MB = 4, 128, 40, 4
    g = workloads.rng(6)
    pool = kvc.Pool(N, MB)
    model = PoolModel(N, 16, MB)
    layer = kvc.PagedLayer.empty(N, H, D, "f16", device=d, fill=float("nan"))
    ref = PagedCache(N, H, D, "f16", fill=np.nan)
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
        ref.write(slots, k, v)
        tables, tl = pool.block_table(seqs)
        q = workloads.normal(g, (4, H, D), "f16")
        got = kvc.append_decode_paged(to_dev(q, d), layer, to_dev(tables, d), to_dev(tl, d),
                                      to_dev(k, d), to_dev(v, d), int(tl.max()),
                                      scale=scale_of(D), workspace=ws)
        if step in (0, 11, 29):
            check(got.float().cpu().numpy(), ref.decode(q, tables, tl, scale_of(D)), 2e-3,
                  f"step {step}")
    assert n_copies == 3
    _compare_pools(layer, ref)


def test_fused_two_phase_and_refusals():
    d = dev()
    note("append-decode two-phase and refusals")
    D, H = 128, 4
    lens = [300, 7, 1000]
    prior = [L - 1 for L in lens]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, prior, H=H, seed=8)
    pool.append(seqs, 1)
    tables, tl = pool.block_table(seqs)
    tdv, tlv = to_dev(tables, d), to_dev(tl, d)
    q = to_dev(workloads.normal(g, (3, H, D), "f16"), d)
    kd = to_dev(workloads.normal(g, (3, H, D), "f16"), d)
    vd = to_dev(workloads.normal(g, (3, H, D), "f16"), d)
    other = _clone_layer(layer)
    a = kvc.append_decode_paged(q, layer, tdv, tlv, kd, vd, 1000)
    out, ws = kvc.append_decode_partial_paged(q, other, tdv, tlv, kd, vd, 1000)
    kvc.decode_merge(3, H, D, out, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, out)
    assert torch.equal(layer.k_pool.view(torch.int16), other.k_pool.view(torch.int16))
    assert torch.equal(layer.v_pool.view(torch.int16), other.v_pool.view(torch.int16))
    # e4m3 caches keep the separate writer (the block scale may have to grow)
    f8 = kvc.PagedLayer.empty(layer.num_blocks, H, D, "e4m3", device=d)
    k8 = torch.zeros((3, H, D), dtype=torch.uint8, device=d)
    with pytest.raises(kvc.KvcError, match="UNSUPPORTED"):
        kvc.append_decode_paged(q, f8, tdv, tlv, k8, k8, 1000)
    # misaligned new rows are refused before any launch
    flat = torch.zeros(3 * H * D + 1, dtype=torch.float16, device=d)
    bad = flat[1:].view(3, H, D)
    with pytest.raises(kvc.KvcError, match="INVALID"):
        kvc.append_decode_paged(q, layer, tdv, tlv, bad, bad, 1000)


# (dtype, D, G): fp16 runs the matrix-core kernel (G = 32 splits each group into two pairs of
# 16 query heads that share the K/V tile); fp32 runs one query head per wavefront (G pairs per
# K/V head). Either way the new row is stored once and every pair scores it from k_new/v_new.
GQA_CASES = [("f16", 128, 2), ("f16", 128, 8), ("f16", 64, 3), ("f16", 128, 32), ("f32", 64, 4)]


@pytest.mark.parametrize("dtype,D,G", GQA_CASES)
def test_paged_gqa_fused_equals_write_then_decode(dtype, D, G):
    d = dev()
    note(f"append-decode gqa paged {dtype} D={D} G={G}")
    H = 2
    prior = [max(L - 1, 0) for L in LENS]
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, dtype, D, prior, H=H, seed=D + G)
    live = [s for s, L in zip(seqs, LENS) if L > 0]
    slots, src, dst = pool.append(live, 1)
    ms, cow = model.append(live, 1)
    assert list(slots) == ms and not cow
    tables, tl = pool.block_table(seqs)
    assert list(tl) == LENS
    B = len(LENS)
    k_new = workloads.normal(g, (B, H, D), dtype)
    v_new = workloads.normal(g, (B, H, D), dtype)
    q = workloads.normal(g, (B, H * G, D), dtype)
    rows = [b for b, L in enumerate(LENS) if L > 0]
    ref.write(slots, k_new[rows], v_new[rows])
    tdv, tlv = to_dev(tables, d), to_dev(tl, d)
    qd, kd, vd = to_dev(q, d), to_dev(k_new, d), to_dev(v_new, d)
    other = _clone_layer(layer)
    fused = kvc.append_decode_gqa_paged(qd, layer, tdv, tlv, kd, vd, max(LENS), scale=scale_of(D))
    kvc.write_paged(other, to_dev(slots, d), to_dev(k_new[rows], d), to_dev(v_new[rows], d))
    plain = kvc.decode_gqa_paged(qd, other, tdv, tlv, max(LENS), scale=scale_of(D))
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    assert torch.equal(layer.k_pool.view(torch.int8), other.k_pool.view(torch.int8))
    assert torch.equal(layer.v_pool.view(torch.int8), other.v_pool.view(torch.int8))
    _compare_pools(layer, ref)
    check(fused.float().cpu().numpy(), ref.decode(q, tables, tl, scale_of(D)), TOL[dtype])
    assert fused[LENS.index(0)].float().abs().sum().item() == 0.0


@pytest.mark.parametrize("dtype,D,G", [("f16", 128, 8), ("f16", 128, 32), ("f32", 64, 4)])
def test_contig_gqa_fused_equals_append_then_decode(dtype, D, G):
    d = dev()
    note(f"append-decode gqa contig {dtype} D={D} G={G}")
    H, S = 2, 528
    B = len(LENS)
    g = workloads.rng(300 + D + G)
    K = workloads.normal(g, (B, S, H, D), dtype)
    V = workloads.normal(g, (B, S, H, D), dtype)
    q = workloads.normal(g, (B, H * G, D), dtype)
    ref = ContigCache(B, H, S, D, dtype, fill=np.nan)
    kc = torch.full((B, H, S, D), float("nan"), dtype=TD[dtype], device=d)
    vc = torch.full_like(kc, float("nan"))
    for b, L in enumerate(LENS):           # prefill positions [0, L-1)
        if L > 1:
            p = np.full(B, S, np.int32)
            p[b] = 0
            kvc.append_contig(kc, vc, to_dev(p, d), to_dev(K[:, :L - 1], d),
                              to_dev(V[:, :L - 1], d))
            ref.append(p, K[:, :L - 1], V[:, :L - 1])
    pos = np.array([L - 1 if L > 0 else S for L in LENS], np.int32)
    k_new, v_new = K[np.arange(B), np.maximum(pos, 0) % S], V[np.arange(B), np.maximum(pos, 0) % S]
    ref.append(pos, k_new[:, None], v_new[:, None])
    kc2, vc2 = kc.clone(), vc.clone()
    lens = to_dev(np.array(LENS, np.int32), d)
    qd, kd, vd = to_dev(q, d), to_dev(k_new, d), to_dev(v_new, d)
    fused = kvc.append_decode_gqa_contig(qd, kc, vc, lens, kd, vd, max(LENS), scale=scale_of(D))
    kvc.append_contig(kc2, vc2, to_dev(pos, d), kd[:, None].contiguous(), vd[:, None].contiguous())
    plain = kvc.decode_gqa_contig(qd, kc2, vc2, lens, max(LENS), scale=scale_of(D))
    torch.cuda.synchronize()
    assert torch.equal(fused, plain)
    np.testing.assert_array_equal(kc.cpu().numpy(), ref.K)
    np.testing.assert_array_equal(vc.cpu().numpy(), ref.V)
    check(fused.float().cpu().numpy(), ref.decode(q, LENS, scale_of(D)), TOL[dtype])


def test_gqa_fused_refusals():
    """8-bit caches refuse the fused call (their block scale may change); k_new of the wrong
    head count is refused by the binding."""
    d = dev()
    note("append-decode gqa refusals")
    H, D, G = 2, 128, 4
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "e4m3", D, [5, 9], H=H, seed=3)
    tables, tl = pool.block_table(seqs)
    q = to_dev(workloads.normal(g, (2, H * G, D), "f16"), d)
    kn = torch.zeros((2, H, D), dtype=layer.k_pool.dtype, device=d)   # codes of the cache dtype
    with pytest.raises(kvc.KvcError):
        kvc.append_decode_gqa_paged(q, layer, to_dev(tables, d), to_dev(tl, d), kn, kn.clone(), 9)
    g, pool, model, seqs, layer, ref, data = _paged_setup(d, "f16", D, [5, 9], H=H, seed=4)
    tables, tl = pool.block_table(seqs)
    wrong = to_dev(workloads.normal(g, (2, H * G, D), "f16"), d)
    with pytest.raises(ValueError):
        kvc.append_decode_gqa_paged(q, layer, to_dev(tables, d), to_dev(tl, d), wrong,
                                    wrong.clone(), 9)
